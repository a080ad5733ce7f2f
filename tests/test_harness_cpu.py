"""CPU tests of the schedule fuzzer and the verdict core (no GPU).

The runner drives a deterministic mock backend that keeps a paged "KV"
state: the value stored for position p is a hash of the token at p and the
value at p-1, and a step's logits row is derived from the value at the
row's position.  Invariant by construction -- unless its divergence knob
mixes the step's batch size into the logits, which must turn the verdict
RED.  Preemption with swap and with recompute must reproduce the same state.
"""
import hashlib
import json
import os

import numpy as np
import pytest

from invariant_bi_rmsnorm_amd import harness as H


class MockBackend:
    page_size = 4

    def __init__(self, num_pages=400, divergence=False):
        self.num_pages = num_pages
        self.kv = np.zeros((num_pages, self.page_size), dtype=np.uint64)
        self.divergence = divergence
        self.steps = 0
        self.batch_sizes = []

    def _h(self, *vals):
        d = hashlib.blake2b(repr(vals).encode(), digest_size=8).digest()
        return np.uint64(int.from_bytes(d, "little"))

    def step(self, segs):
        self.steps += 1
        self.batch_sizes.append(len(segs))
        rows, toks = [], []
        for s in segs:
            for j, t in enumerate(s.tokens):
                p = s.pos0 + j
                prev = np.uint64(0) if p == 0 else self.kv[s.pages[(p - 1) // 4], (p - 1) % 4]
                self.kv[s.pages[p // 4], p % 4] = self._h(int(t), p, int(prev))
            if s.want_logits:
                p = s.pos0 + len(s.tokens) - 1
                v = int(self.kv[s.pages[p // 4], p % 4])
                logits = np.frombuffer(hashlib.sha256(v.to_bytes(8, "little")).digest(),
                                       dtype=np.uint8).astype(np.float32)
                if self.divergence and len(segs) > 1:
                    logits[0] += 1.0   # a batch-dependent rounding, caricatured
                rows.append(logits.tobytes())
                toks.append(int(np.argmax(logits)) % 50)
        return rows, toks

    def swap_out(self, pages):
        return self.kv[pages].copy()

    def swap_in(self, blob, pages):
        self.kv[pages[:len(blob)]] = blob


def make_reqs(n=8, seed=0):
    rng = np.random.default_rng(seed)
    return [H.Request(i, list(rng.integers(0, 50, size=int(rng.integers(1, 30)))),
                      int(rng.integers(1, 12))) for i in range(n)]


def test_verdict_core_pure():
    base = {0: {3: "a", 4: "b"}, 1: {1: "c"}}
    same = [{0: {3: "a", 4: "b"}, 1: {1: "c"}}] * 3
    rep = H.diff_runs(base, same)
    assert rep["divergent"] == {} and rep["compared"] == 9 and rep["unique_samples_max"] == 1
    out = H.decide(rep, {0: 2, 1: 1}, {0: True, 1: True}, 2)
    assert out["verdict"] == H.GREEN and out["rule_of_three_upper"] == pytest.approx(3 / 9)
    bad = [{0: {3: "a", 4: "x"}, 1: {1: "c"}}]
    rep = H.diff_runs(base, bad)
    assert rep["divergent"] == {0: 1} and rep["unique_samples_max"] == 2
    assert H.decide(rep, {0: 1, 1: 1}, {0: True, 1: True}, 2)["verdict"] == H.RED
    # a clean run that never co-batched a request earns nothing
    rep = H.diff_runs(base, same)
    assert H.decide(rep, {0: 1, 1: 0}, {0: True, 1: True}, 2)["verdict"] == H.UNVERIFIED
    # an incomplete request earns nothing
    assert H.decide(rep, {0: 1, 1: 1}, {0: True, 1: False}, 2)["verdict"] == H.UNVERIFIED
    # missing records earn nothing
    rep = H.diff_runs(base, [{0: {3: "a"}, 1: {1: "c"}}])
    assert H.decide(rep, {0: 1, 1: 1}, {0: True, 1: True}, 2)["verdict"] == H.UNVERIFIED


def test_fuzzed_schedules_green_on_invariant_backend(tmp_path):
    reqs = make_reqs(10, seed=1)
    path = os.path.join(tmp_path, "cert.json")
    fz = H.FuzzConfig(seed=7, max_rows=24, max_reqs=6, p_preempt=0.3, p_swap=0.5)
    out = H.verify(lambda: MockBackend(), reqs, n_schedules=6, fuzz=fz, report_path=path)
    assert out["verdict"] == H.GREEN, out
    assert out["cobatch_frac"] == 1.0 and out["completion_frac"] == 1.0
    assert out["rerecord_mismatch"] == 0
    with open(path) as f:
        assert json.load(f)["verdict"] == H.GREEN


def test_fuzzed_schedules_red_on_batch_dependent_backend():
    reqs = make_reqs(8, seed=2)
    fz = H.FuzzConfig(seed=3, max_rows=24, max_reqs=6, p_preempt=0.2)
    out = H.verify(lambda: MockBackend(divergence=True), reqs, n_schedules=3, fuzz=fz)
    assert out["verdict"] == H.RED
    assert out["divergent_requests"] > 0


def test_schedules_actually_vary_and_preempt():
    reqs = make_reqs(10, seed=4)
    sizes, preempts, cuts = set(), 0, set()
    for seed in range(5):
        be = MockBackend()
        runner = H.Runner(be, reqs, H.FuzzConfig(seed=seed, max_rows=24, max_reqs=6,
                                                 p_preempt=0.4))
        orig = runner._preempt
        count = [0]

        def spy(r, orig=orig, count=count):
            count[0] += 1
            orig(r)
        runner._preempt = spy
        runner.run()
        sizes |= set(be.batch_sizes)
        preempts += count[0]
    assert len(sizes) >= 4          # compositions of several sizes
    assert preempts > 0             # preemption (swap or recompute) happened


def test_alone_baseline_runs_one_request_per_step():
    be = MockBackend()
    H.Runner(be, make_reqs(5, seed=5), H.FuzzConfig(alone=True, prefill_whole=True)).run()
    assert set(be.batch_sizes) == {1}


def test_report_write_is_atomic(tmp_path):
    p = os.path.join(tmp_path, "sub", "r.json")
    H.write_report(p, {"verdict": "GREEN", "n": 1})
    H.write_report(p, {"verdict": "RED", "n": 2})
    with open(p) as f:
        assert json.load(f) == {"verdict": "RED", "n": 2}
    assert [x for x in os.listdir(os.path.dirname(p)) if x.endswith(".tmp")] == []


# ---------------------------------------------------------------------------
# decode-verify-rollback (protocol logic on mock engines)
# ---------------------------------------------------------------------------

class MockEngine:
    """Engine-shaped mock over a shared token store: the value at position p
    hashes the token at p with the value at p - 1, and a row's next token is
    that value mod V.  noise > 0 makes it a 'fast path': with that
    probability (drawn from the position, the batch size and a step counter)
    a row's token is bumped by one -- a batch-dependent flip."""

    V = 50

    def __init__(self, store, noise=0.0):
        self.store, self.noise, self.steps = store, noise, 0

    def _h(self, *vals):
        d = hashlib.blake2b(repr(vals).encode(), digest_size=8).digest()
        return int.from_bytes(d, "little")

    def step(self, segs):
        import torch
        from invariant_bi_rmsnorm_amd.model import StepOutput
        self.steps += 1
        order = [i for i, s in enumerate(segs) if len(s.tokens) == 1] + \
                [i for i, s in enumerate(segs) if len(s.tokens) > 1]
        toks, seg_index = [], []
        for i in order:
            s = segs[i]
            key = tuple(s.pages)
            for j, t in enumerate(s.tokens):
                p = s.pos0 + j
                prev = self.store.get((key, p - 1), 0)
                self.store[(key, p)] = self._h(t, prev)
                if s.all_logits or (s.want_logits and j == len(s.tokens) - 1):
                    tok = self.store[(key, p)] % self.V
                    if self.noise and (self._h(p, len(segs), self.steps) % 1000) < 1000 * self.noise:
                        tok = (tok + 1) % self.V
                    toks.append(tok)
                    seg_index.append(i)
        t = torch.tensor(toks, dtype=torch.int32)
        return StepOutput(torch.zeros((len(toks), 1)), t, seg_index)


@pytest.mark.parametrize("noise,window,group", [(0.0, 8, 2), (0.05, 8, 2), (0.3, 5, 3),
                                                (0.05, 64, 8)])
def test_decode_verify_rollback_commits_the_verifier_sequence(noise, window, group):
    rng = np.random.default_rng(7)
    prompts = [list(rng.integers(0, 50, int(rng.integers(1, 30)))) for _ in range(6)]
    pages = [[1000 + r] for r in range(6)]          # one 'page' list per request
    ref = H.greedy_decode(MockEngine({}), prompts, pages, max_new=70, chunk=7)
    store = {}
    out, st = H.decode_verify_rollback(MockEngine(store, noise), MockEngine(store), prompts,
                                       pages, max_new=70, window=window, group=group, chunk=7)
    assert [o[:70] for o in out] == [r[:70] for r in ref]
    assert all(len(o) == 70 for o in out)
    if noise == 0.0:
        assert st.mismatches == 0 and st.discarded == 0
    else:
        assert st.mismatches > 0 and st.discarded > 0
    assert st.committed == sum(len(o) - 1 for o in out)
    # the fast path alone does drift from the verifier's sequence
    if noise >= 0.05:
        fast_only = H.greedy_decode(MockEngine({}, noise), prompts, pages, max_new=70, chunk=7)
        assert fast_only != ref


def test_full_batch_schedules_and_config_list():
    """p_full = 1 with all arrivals at once puts every request in one step
    (batch 1 in the baseline vs all of them here), the rows shared out so
    that no segment is dropped; a list of configs runs one schedule each;
    preemptions by swap and by recompute are both counted."""
    reqs = make_reqs(12, seed=4)
    for r in reqs:
        r.max_new = max(r.max_new, 4)
    full = H.FuzzConfig(seed=5, max_rows=64, max_reqs=64, p_preempt=0.0, p_full=1.0,
                        arrival_steps=1)
    mixed = H.FuzzConfig(seed=6, max_rows=64, max_reqs=64, p_preempt=0.6, p_swap=0.5,
                         p_full=0.3)
    out = H.verify(lambda: MockBackend(), reqs, n_schedules=0, fuzz=[full, mixed])
    assert out["verdict"] == H.GREEN, out
    assert out["schedules"] == 2 and out["schedule_seeds"] == [5, 6]
    assert out["max_requests_per_step"] == len(reqs)
    assert out["max_rows_per_step"] <= 64
    assert out["preemptions"]["swap"] > 0 and out["preemptions"]["recompute"] > 0
    out = H.verify(lambda: MockBackend(divergence=True), reqs, n_schedules=0, fuzz=[full])
    assert out["verdict"] == H.RED
