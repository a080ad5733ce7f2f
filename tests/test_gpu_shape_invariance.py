"""Bitwise batch invariance of the composed engine at the Llama-3-8B shape.

"Lockstep", section "Proving it": every schedule a scheduler may produce
(composition, row order, arrival, preemption and readmission) must give each
request the logits of the request run alone, bit for bit.

- One full-shape decoder layer (d 4096, 32/8 heads of 128, SwiGLU 14336,
  vocab 128256, 256-key chunks, bf16 weights N(0, 0.02), KV history N(0, 1)
  with lengths uniform 32..4096 in scattered pages): 128 requests each run
  alone, then drawn in random mixes and row orders at batch 1, 7, 32 and 64;
  every request's fp32 logits row must equal its alone row bit for bit.  Two
  requests of a batch-64 mix are checked against the oracle kernel by kernel
  on the engine's own inputs (tests/layer_check.py), with the LM head gate.
- The whole 32-layer model under the schedule fuzzer: 64 requests, prompts
  uniform 32..1024 tokens, 4 greedy tokens each; fuzzed compositions up to
  all 64 requests in one step (batch 1 in the baseline vs 64), random
  chunked-prefill cuts in steps of up to 4096 rows, arrival order, and
  preemption with readmission by swap and by recompute -- GREEN.  The same
  fuzzer over the batch-adaptive twins must find divergent requests (RED).

Prompts are bounded at 1024 tokens here (the workload's own lengths reach
4096) so the 32-layer fuzz finishes in a few minutes.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import dev

pytestmark = pytest.mark.gpu
L = pytest.importorskip("invariant_bi_rmsnorm_amd._lib")
from invariant_bi_rmsnorm_amd import harness as H  # noqa: E402
from invariant_bi_rmsnorm_amd.model import (LLAMA3_8B, Engine, KVPool, Segment,  # noqa: E402
                                            init_weights)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


@pytest.mark.timeout(900)
def test_single_full_layer_batches_1_7_32_64_bitwise_and_oracle():
    from layer_check import check_layer, layer_taps, tap_rows
    import oracle.llama as OL
    cfg = replace(LLAMA3_8B, layers=1)
    n_pool = 128
    w = init_weights(cfg, 51, dev(), source="device")
    lens = synth.uniform_lengths(n_pool, 32, 4096, seed=52)
    place = synth.scatter_pages(lens, cfg.page_size, seed=53)
    pool = KVPool(cfg, place.num_pages, dev())
    g = torch.Generator(device=dev()).manual_seed(54)
    pool.k.normal_(generator=g)
    pool.v.normal_(generator=g)
    eng = Engine(cfg, w, pool, dev(), max_rows=64, max_pages_per_req=place.max_pages + 1)
    toks = synth.token_ids(n_pool, cfg.vocab, seed=55)

    def seg(r):
        npg = (int(lens[r]) + cfg.page_size - 1) // cfg.page_size
        return Segment(pages=[int(p) for p in place.block_table[r, :npg]],
                       pos0=int(lens[r]) - 1, tokens=[int(toks[r])])

    alone = []
    for r in range(n_pool):
        out = eng.step([seg(r)])
        alone.append(_bits(out.logits[0].cpu().numpy()))
    rng = np.random.default_rng(56)
    checked = 0
    for B, trials in ((1, 4), (7, 4), (32, 3), (64, 3)):
        for trial in range(trials):
            rows = [int(r) for r in rng.choice(n_pool, size=B, replace=False)]
            out = eng.step([seg(r) for r in rows])
            got = out.logits.cpu().numpy()
            for k, si in enumerate(out.seg_index):
                r = rows[si]
                assert np.array_equal(_bits(got[k]), alone[r]), \
                    f"batch {B} trial {trial}: request {r} differs from alone"
                checked += 1
    print(f"{checked} request rows bit-identical to alone over batches 1/7/32/64")
    # oracle tolerance: two requests of a batch-64 mix, kernel by kernel
    rows = [int(r) for r in rng.choice(n_pool, size=64, replace=False)]
    segs = [seg(r) for r in rows]
    pick = [int(np.argmin(lens[rows])), int(np.argmax(lens[rows]))]   # indices into rows
    m = eng.upload(eng.pack(segs))
    packed = [m["order"].index(i) for i in pick]
    tap, store = tap_rows(packed)
    out = eng.forward(m, tap=tap)
    torch.cuda.synchronize()
    for i, si in enumerate(pick):           # the logits are the alone bits as well
        k = out.seg_index.index(si)
        assert np.array_equal(_bits(out.logits[k].cpu().numpy()), alone[rows[si]])
    om = OL.OracleModel(cfg, w, num_pages=1, cos_t=eng.cos.cpu(), sin_t=eng.sin.cpu())
    kps, vps, pos = [], [], []
    for si in pick:
        idx = torch.tensor(segs[si].pages, device=dev())
        kps.append(L.k_pool_to_rows(pool.k[0, idx]).float().cpu().numpy())
        vps.append(pool.v[0, idx].float().cpu().numpy())
        pos.append(segs[si].pos0)
    rep = check_layer(cfg, om.layers[0], layer_taps(store, 0), 0, pos, kps, vps, om.cos, om.sin)
    print("per-kernel max error / bound:", {k_: round(v_, 3) for k_, v_ in rep.items()})
    lo = oracle.gemm(store[("x_final", 1)], om.lm_head, False)
    for i, si in enumerate(pick):
        gl = out.logits[out.seg_index.index(si)].cpu().numpy()
        e = float(np.max(np.abs(gl - lo[i])) / np.max(np.abs(lo[i])))
        assert e <= 2e-3, f"request {rows[si]}: LM head rel err {e}"
        assert int(np.argmax(gl)) == int(np.argmax(lo[i]))


def _fuzz_requests(n, seed, lo=32, hi=1024, max_new=4):
    lens = synth.uniform_lengths(n, lo, hi, seed=seed)
    return [H.Request(i, [int(t) for t in synth.token_ids(int(lens[i]), LLAMA3_8B.vocab,
                                                           seed=seed + 1 + i)], max_new)
            for i in range(n)]


def _backend_factory(w, reqs, free):
    cfg = LLAMA3_8B
    need = sum(-(-(len(r.prompt) + r.max_new) // cfg.page_size) for r in reqs)
    num_pages = int(need * 1.25) + 8
    max_pages = max(-(-(len(r.prompt) + r.max_new) // cfg.page_size) for r in reqs) + 1

    def fresh():
        pool = KVPool(cfg, num_pages, dev())
        return H.EngineBackend(Engine(cfg, w, pool, dev(), max_rows=256,
                                      max_pages_per_req=max_pages, free=free))
    return fresh


@pytest.fixture(scope="module")
def llama_weights():
    w = init_weights(LLAMA3_8B, 61, dev(), source="device")
    yield w
    del w
    torch.cuda.empty_cache()


@pytest.mark.timeout(1200)
def test_llama8b_fuzzed_schedules_green(llama_weights):
    reqs = _fuzz_requests(64, seed=700)
    # one schedule of full batches (every request in every step, chunked
    # prefill cuts, no preemption: batch-64 decode steps), two fully fuzzed
    full = H.FuzzConfig(seed=71, max_rows=4096, max_reqs=64, p_preempt=0.0, p_full=1.0,
                        arrival_steps=3)
    mixed = [H.FuzzConfig(seed=s, max_rows=4096, max_reqs=64, p_preempt=0.25, p_swap=0.5,
                          p_full=0.3, arrival_steps=6) for s in (72, 73)]
    out = H.verify(_backend_factory(llama_weights, reqs, free=False), reqs, n_schedules=0,
                   fuzz=[full] + mixed)
    print({k: out[k] for k in ("verdict", "compared", "cobatch_frac", "max_requests_per_step",
                               "max_rows_per_step", "preemptions", "rule_of_three_upper")})
    assert out["verdict"] == H.GREEN, out
    assert out["max_requests_per_step"] == 64          # batch 1 (baseline) vs 64
    assert out["preemptions"]["swap"] > 0 and out["preemptions"]["recompute"] > 0, out


@pytest.mark.timeout(900)
def test_llama8b_fuzzed_schedules_red_on_twins(llama_weights):
    reqs = _fuzz_requests(16, seed=800, lo=300, hi=1024, max_new=3)
    fz = H.FuzzConfig(seed=81, max_rows=4096, max_reqs=16, p_preempt=0.0, p_full=0.5,
                      arrival_steps=2)
    out = H.verify(_backend_factory(llama_weights, reqs, free=True), reqs, n_schedules=1,
                   fuzz=fz)
    print({k: out[k] for k in ("verdict", "divergent_requests", "compared",
                               "max_requests_per_step")})
    assert out["verdict"] == H.RED, out
    assert out["divergent_requests"] > 0
