#!/usr/bin/env python3
"""Decode throughput of the batch-invariant path on one MI355X.

Workload (one "step"): a decode step of a 32-layer Llama-3-8B-shaped model
(d 4096, 32/8 heads of 128, SwiGLU 14336, vocab 128256, bf16 weights
N(0, 0.02) drawn on the device) for a batch of 64 requests whose KV lengths
are uniform in 32..4096 (seeded), KV history N(0, 1) in 16-token pages
scattered over a pool 1.25x the live pages.  Every kernel of the step is a
libbi.so call: per layer RMSNorm, QKV GEMM, RoPE + KV append, split-KV
decode attention, serial merge, O GEMM, add, RMSNorm, gate/up GEMM,
SiLU-mul, down GEMM, add; then RMSNorm, LM-head GEMM (fp32 logits), argmax.
The KV lengths stay fixed across timed steps (each step rewrites the slot of
the token it decodes), so every step does the same work.

Prints one JSON line.  `value` = decode tokens/s of the whole step (the
step is captured in a HIP graph and replayed; the graph's logits are
checked bitwise against an eager step first).  The same step on the tuned
batch-adaptive twin (the engine's "tuned" mode: at every call site the
fastest of the invariant configuration and the batch-adaptive ones --
split-K GEMMs, 64-key KV chunks, occupancy-driven KV splits, norms split
over workgroups -- measured per shape on first use) is timed the same way,
graph-replayed, over the same KV pool and weights:
`invariance_overhead_pct` = invariant step time / twin step time - 1,
with the twin's choices and per-kernel deltas.  `sweep` repeats both at
other batch sizes (1, 7, 32 by default).  `roofline` is for the
kernel with the largest share of step time in a second timed region of eager
steps (HIP event pairs on the launch stream around every kernel); its
duration is then taken from back-to-back launches of the step's last-layer
instance between one event pair, which leaves out each pair's own cost; its algorithmic
bytes are those of algorithmic_bytes() below (the least a launch must
move: KV of every live token, q, partials; or weights plus activations).  `cpu_baseline` times the CPU oracle on a
bounded sample (all requests of the step through as many decoder layers
as fit in about ten seconds, plus the LM head) and scales it to the full
step.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # B/s, MI355X
BF16_PEAK = 2.5e15         # FLOP/s dense MFMA
METRIC = "decode tokens/s @Llama-3-8B shape, batch 1–64; HBM GB/s % peak; invariance overhead %"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", default="1,7,32", help="extra batch sizes ('' for none)")
    ap.add_argument("--only", default="",
                    help="time one kernel of the step instead (decode_attn, merge, ...; a "
                         "comma list of gemm_qkv, gemm_o, gemm_gate_up, gemm_down for the "
                         "projection GEMMs over the weights of all layers in turn; "
                         "'decode_attn_long' for paged decode attention at KV lengths "
                         "log-uniform 128..32768; 'prefill_gemm'; 'log_softmax' / 'sample' for "
                         "logprobs / seeded draws over the batch's logits; or 'copy' for a "
                         "plain 1 GiB device copy), e.g. under rocprofv3 --pmc")
    ap.add_argument("--twin", action="store_true", help="with --only: the twin's kernel")
    ap.add_argument("--twin-mode", default="tuned", choices=("tuned", "free"),
                    help="with --only --twin: the tuned twin (fastest configuration per "
                         "site) or the all-adaptive one")
    ap.add_argument("--launches", type=int, default=50)
    ap.add_argument("--prompt", type=int, default=2048, help="with --only prefill_attn")
    ap.add_argument("--oracle-table", action="store_true",
                    help="time the CPU oracle beside the GPU kernels on the decode-attention "
                         "(batch 1 and 64, long contexts), M=513 GEMM and prefill-attention "
                         "workloads")
    ap.add_argument("--dvr", action="store_true",
                    help="decode-verify-rollback (twins decode, invariant kernels verify) "
                         "against greedy decoding on each engine alone; eager steps")
    ap.add_argument("--dvr-new", type=int, default=256, help="with --dvr: tokens per request")
    ap.add_argument("--dvr-window", type=int, default=64)
    ap.add_argument("--dvr-group", type=int, default=8)
    ap.add_argument("--traffic-summary", default="",
                    help="summarise rocprofv3 --pmc runs (FETCH_SIZE / WRITE_SIZE of --only "
                         "decode_attn and of --only copy) found under this directory")
    ap.add_argument("--gemm-counters-summary", default="",
                    help="summarise rocprofv3 --pmc passes of --only gemm_qkv,gemm_o,"
                         "gemm_gate_up,gemm_down (one subdirectory per pass) found under this "
                         "directory")
    ap.add_argument("--mfma-summary", default="",
                    help="summarise a rocprofv3 --pmc run of --only prefill_gemm "
                         "(SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16, "
                         "GRBM_GUI_ACTIVE) found under this directory")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def model_config(args):
    from dataclasses import replace
    from invariant_bi_rmsnorm_amd.model import LLAMA3_8B
    return replace(LLAMA3_8B, layers=args.layers)


def build_workload(args, B, torch, dev, w, free=False, twin_mode="tuned"):
    """KV pool, engine(s) and the packed decode step for batch B; free=True
    also builds a twin engine (mode twin_mode: "tuned", the fair
    batch-adaptive baseline, or "free", every kernel on its twin) over the
    same pool."""
    import synth
    from invariant_bi_rmsnorm_amd.model import Engine, KVPool, Segment
    cfg = model_config(args)
    kv_len = synth.uniform_lengths(B, 32, 4096, seed=args.seed + 11)
    place = synth.scatter_pages(kv_len, cfg.page_size, seed=args.seed + 12)
    pool = KVPool(cfg, place.num_pages, dev)
    g = torch.Generator(device=dev).manual_seed(args.seed + 13)
    for li in range(cfg.layers):
        pool.k[li].normal_(generator=g)
        pool.v[li].normal_(generator=g)
    eng = Engine(cfg, w, pool, dev, max_rows=B, max_pages_per_req=max(place.max_pages, 257))
    twin = Engine(cfg, w, pool, dev, max_rows=B, max_pages_per_req=max(place.max_pages, 257),
                  mode=twin_mode) if free else None
    toks = synth.token_ids(B, cfg.vocab, seed=args.seed + 15)
    segs = []
    for r in range(B):
        npg = (int(kv_len[r]) + cfg.page_size - 1) // cfg.page_size
        segs.append(Segment(pages=[int(p) for p in place.block_table[r, :npg]],
                            pos0=int(kv_len[r]) - 1, tokens=[int(toks[r])]))
    meta = eng.upload(eng.pack(segs))
    tmeta = twin.upload(twin.pack(segs)) if free else None
    return cfg, eng, twin, meta, kv_len, place, tmeta


def algorithmic_bytes(name, cfg, B, kv_len, meta):
    """Bytes one launch must move at minimum: decode attention reads K and V
    of every live token (h_kv * d_h * 2 bytes each, twice), q, and writes
    and the merge re-reads the fp32 partials; a GEMM reads W [N, K] and A
    [M, K] once and writes C [M, N] (the gate/up product writes its SwiGLU
    activation, [M, N/2])."""
    if name == "decode_attn":
        kv = int(sum(kv_len)) * cfg.h_kv * cfg.d_h * 2 * 2
        q = B * cfg.h * cfg.d_h * 2
        part = meta["total_chunks"] * cfg.h * (cfg.d_h + 2) * 4
        return kv + q + part
    shapes = {"gemm_qkv": (cfg.qkv_out, cfg.d), "gemm_o": (cfg.d, cfg.h * cfg.d_h),
              "gemm_gate_up": (2 * cfg.ffn, cfg.d), "gemm_down": (cfg.d, cfg.ffn),
              "gemm_lm_head": (cfg.vocab, cfg.d)}
    if name in shapes:
        N, K = shapes[name]
        out_b = 4 if name == "gemm_lm_head" else 2
        out_n = N // 2 if name == "gemm_gate_up" else N
        return 2 * N * K + 2 * B * K + out_b * B * out_n
    if name == "merge":
        return meta["total_chunks"] * cfg.h * (cfg.d_h + 2) * 4 + B * cfg.h * cfg.d_h * 2
    return None


def time_steps(eng, meta, steps, torch, graph):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if graph is not None:
            graph.replay()
        else:
            eng.forward(meta)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def capture(eng, meta, torch, warmup, exact=True):
    """Eager warmup, then the step captured in a HIP graph; the graph's
    logits must equal an eager step's over several replays with eager work
    in between -- bit for bit (exact), or, for a twin whose kernels need not
    repeat their bits, within 1e-3 of the largest logit -- else the eager
    step is timed.  Returns (graph or None, check result)."""
    for _ in range(max(warmup, 1)):
        ref = eng.forward(meta)
    torch.cuda.synchronize()
    ref_logits = ref.logits.clone()
    try:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                out = eng.forward(meta)
        torch.cuda.current_stream().wait_stream(s)
        same = True
        for _ in range(3):
            graph.replay()
            torch.cuda.synchronize()
            if exact:
                same &= bool(torch.equal(out.logits.view(torch.int32),
                                         ref_logits.view(torch.int32)))
            else:
                err = (out.logits - ref_logits).abs().max() / ref_logits.abs().max()
                same &= bool(err <= 1e-3)
            eng.forward(meta)          # eager work between replays
            torch.cuda.synchronize()
        if not same:
            log("graph replay differs from the eager step; timing eager")
            return None, False
        return graph, True
    except Exception as e:  # capture unsupported -> eager timing
        log(f"graph capture failed ({e}); timing eager")
        return None, None


def per_kernel_times(eng, meta, steps, torch):
    """Eager steps with a HIP event pair around every kernel, on the stream
    the kernels are launched on.  A short device spin before each start
    event keeps the GPU busy while the host enqueues the event and the
    kernel, so host launch gaps stay out of the measured interval."""
    events, grab = {}, {}

    spin = getattr(torch.cuda, "_sleep", None)

    def timer(name, fn):
        if spin is not None:
            spin(600000)   # ~250 us: the host is well ahead when the events land
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        events.setdefault(name, []).append((a, b))
        grab[name] = fn                      # the last layer's instance

    torch.cuda.synchronize()
    for _ in range(steps):
        eng.forward(meta, timer=timer)
    torch.cuda.synchronize()
    per = {}
    for name, lst in events.items():
        ms = [a.elapsed_time(b) for a, b in lst]
        per[name] = {"launches_per_step": len(ms) // steps, "avg_us": 1e3 * sum(ms) / len(ms),
                     "total_ms_per_step": sum(ms) / steps}
    return per, grab


def back_to_back_us(fn, torch, launches=20):
    """Average duration of `launches` back-to-back launches of one kernel of
    the step (the last layer's instance, same inputs) between one HIP event
    pair on the launch stream: no per-launch event cost inside."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(launches):
        fn()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / launches


def run_batch(args, B, torch, dev, w, want_detail):
    cfg, eng, twin, meta, kv_len, place, tmeta = build_workload(args, B, torch, dev, w, free=True)
    log(f"B={B}: {int(sum(kv_len))} KV tokens, {meta['total_chunks']} chunks")
    res = {"B": B}
    for tag, e, mm in (("inv", eng, meta), ("free", twin, tmeta)):
        graph, ok = (None, None) if args.no_graph else capture(e, mm, torch, args.warmup,
                                                              exact=(tag == "inv"))
        sec = time_steps(e, mm, args.steps, torch, graph)
        res[tag] = {"ms_per_step": sec * 1e3, "tokens_per_s": B / sec,
                    "graph": graph is not None, "graph_matches_eager": ok}
        del graph
    res["invariance_overhead_pct"] = 100.0 * (res["inv"]["ms_per_step"] /
                                              res["free"]["ms_per_step"] - 1.0)
    res["twin_choices"] = twin_choices(twin)
    step_bytes = (cfg.weight_bytes() - 2 * cfg.vocab * cfg.d
                  + int(sum(kv_len)) * cfg.kv_bytes_per_token())
    res["step_bytes"] = step_bytes
    res["hbm_frac_of_step_bound"] = (step_bytes / (res["inv"]["ms_per_step"] * 1e-3)) / HBM_PEAK
    log(f"B={B}: invariant {res['inv']['ms_per_step']:.3f} ms/step, tuned twin "
        f"{res['free']['ms_per_step']:.3f} ms/step")
    if not want_detail:
        return res, None
    # second timed region: eager steps, HIP events around every kernel
    per, grab = per_kernel_times(eng, meta, args.steps, torch)
    per_free, _ = per_kernel_times(twin, tmeta, args.steps, torch)
    detail = {"per_kernel": per, "per_kernel_free": per_free, "grab": grab, "cfg": cfg,
              "kv_len": kv_len,
              "meta": meta, "eng": eng, "weights": w, "place": place}
    return res, detail


def twin_choices(twin):
    """Which configuration the tuned twin runs at each call site ("inv" =
    the invariant kernel), with the candidates' measured us."""
    labels = {"norm": ("inv", "split rows"), "qkv": ("inv", "split-K"),
              "decode_attn": ("inv C=256", "inv C=64", "occupancy splits"),
              "prefill_attn": ("inv", "cut-relative chunks"), "gemm_o": ("inv", "split-K"),
              "add_norm": ("inv fused", "add + split rows"),
              "norm_qkv": ("inv fused norm", "add + split rows + split-K"),
              "gemm_gate_up": ("inv", "inv unfused", "split-K"),
              "gemm_down": ("inv", "split-K"), "gemm_lm_head": ("inv", "split-K")}
    out = {}
    for key, k in twin.tuner.best.items():
        site = key[0]
        lab = labels.get(site, ())
        times = twin.tuner.times.get(key)
        if site == "gemm_gate_up" and times is not None and len(times) == 2:
            lab = ("inv", "split-K")
        if site == "decode_attn" and times is not None and len(times) == 2:
            lab = ("inv C=256", "occupancy splits")
        out[site] = {"picked": lab[k] if k < len(lab) else k,
                     "candidates_us": dict(zip(lab, times)) if times else None}
    return out


def cpu_baseline(args, detail, B, budget_s=10.0):
    """The oracle on a bounded sample of the same step: all B requests at
    their own KV lengths through decoder layers (layer 0's weights, the
    same work as any layer) until about budget_s seconds have passed, then
    final norm + LM head; scaled to tokens/s of the 32-layer step."""
    import numpy as np
    import oracle
    from oracle.llama import gate_up_halves
    import synth
    cfg, kv_len = detail["cfg"], detail["kv_len"]
    S = B
    lens = kv_len[:S]
    place = synth.scatter_pages(lens, cfg.page_size, seed=args.seed + 21)
    shape = (place.num_pages, cfg.h_kv, cfg.page_size, cfg.d_h)
    kp = synth.normal(shape, seed=args.seed + 22).numpy()
    vp = synth.normal(shape, seed=args.seed + 23).numpy()
    lw = detail["weights"].layers[0]
    W = {k: getattr(lw, k).float().cpu().numpy() for k in
         ("attn_norm", "wqkv", "wo", "ffn_norm", "wgu", "wdown")}
    W["wgu"] = gate_up_halves(W["wgu"])   # [W_g; W_u] out of the 8-row blocks
    lm = detail["weights"].lm_head.float().cpu().numpy()
    fn = detail["weights"].final_norm.float().cpu().numpy()
    cos_t, sin_t = synth.rope_tables(int(lens.max()) + 16, cfg.d_h, cfg.rope_theta)
    h = synth.normal((S, cfg.d), seed=args.seed + 24, std=1.0).numpy()
    pos = lens - 1
    hd, kvd = cfg.h * cfg.d_h, cfg.h_kv * cfg.d_h
    n_layers = 0
    t0 = time.perf_counter()
    while n_layers < cfg.layers and time.perf_counter() - t0 < budget_s:
        x = oracle.rmsnorm(h, W["attn_norm"], cfg.eps, True)
        qkv = oracle.gemm(x, W["wqkv"], True)
        q = oracle.rope(qkv[:, :hd].reshape(S, cfg.h, cfg.d_h), pos, cos_t, sin_t, True)
        k = oracle.rope(qkv[:, hd:hd + kvd].reshape(S, cfg.h_kv, cfg.d_h), pos, cos_t, sin_t,
                        True)
        for r in range(S):
            p = int(pos[r])
            pg = place.block_table[r, p // cfg.page_size]
            kp[pg, :, p % cfg.page_size] = k[r]
            vp[pg, :, p % cfg.page_size] = qkv[r, hd + kvd:].reshape(cfg.h_kv, cfg.d_h)
        a = oracle.decode_attn(q, kp, vp, place.block_table, lens, cfg.h_kv, cfg.page_size,
                               cfg.kv_chunk, cfg.scale, True)
        h = oracle.add(h, oracle.gemm(a.reshape(S, hd), W["wo"], True), True)
        x = oracle.rmsnorm(h, W["ffn_norm"], cfg.eps, True)
        h = oracle.add(h, oracle.gemm(oracle.silu_mul(oracle.gemm(x, W["wgu"], True), True),
                                      W["wdown"], True), True)
        n_layers += 1
    t_layers = time.perf_counter() - t0
    t1 = time.perf_counter()
    logits = oracle.gemm(oracle.rmsnorm(h, fn, cfg.eps, True), lm, False)
    oracle.argmax(logits)
    t_head = time.perf_counter() - t1
    step_s = cfg.layers * t_layers / n_layers + t_head
    return {"value": S / step_s, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"all {S} requests of the step (KV lengths {int(lens.min())}.."
                      f"{int(lens.max())}) through {n_layers} of {cfg.layers} decoder layers "
                      f"({t_layers:.1f} s) plus final norm + LM head ({t_head:.1f} s); layer "
                      f"time scaled to {cfg.layers} layers",
            "sample_seconds": round(t_layers + t_head, 2)}


def prefill_gemm(torch, dev, M=8192, N=14336, K=4096, launches=50, warm=30):
    """The chunked-prefill GEMM: M rows (prefill chunks plus decode rows),
    K 4096 -> N 14336, bf16 in and out, fp32 accumulation.  Timed with HIP
    events on its stream; 2MNK flops against the dense bf16 MFMA peak.  The
    first ten or so back-to-back launches run while the clock is still
    settling (about 850 us each against about 720 us after), so `warm`
    launches go first and `launches` are timed."""
    from invariant_bi_rmsnorm_amd import _lib as L
    g = torch.Generator(device=dev).manual_seed(7)
    A = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    W = L.pack_weight((torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16))
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    for _ in range(warm):
        L.bi_gemm(A, W, C)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(launches):
        L.bi_gemm(A, W, C)
    b.record()
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / launches
    tf = 2.0 * M * N * K / us / 1e6
    return {"kernel": "bi_gemm prefill", "M": M, "N": N, "K": K, "warmup_launches": warm,
            "launches": launches, "avg_us": round(us, 1),
            "TFLOPs": round(tf, 1), "peak": BF16_PEAK / 1e12, "frac": round(tf * 1e12 / BF16_PEAK, 4),
            # rocprofv3 counters of the same launch (profiles/), null once the
            # GEMM sources changed since they were taken
            "counters": measured_mfma()}


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_attn_traffic_llama3_8b_b64.md")
MFMA_PROFILE = os.path.join(ROOT, "profiles", "prefill_gemm_mfma_m8192_n14336_k4096.md")
MFMA_SOURCES = ("invariant_bi_rmsnorm_amd/csrc/gemm.hip", "invariant_bi_rmsnorm_amd/csrc/common.h")
TRAFFIC_SOURCES = ("invariant_bi_rmsnorm_amd/csrc/attention.hip",
                   "invariant_bi_rmsnorm_amd/csrc/common.h")


def kernel_source_hash(sources=None):
    """sha256 over the sources a kernel is built from (by default the
    decode-attention kernel's)."""
    import hashlib
    h = hashlib.sha256()
    for rel in sources or TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _counter_rows(d, counter, match):
    """Per-dispatch values of `counter` for kernels whose name contains
    `match`, from a rocprofv3 --output-format csv run under directory d."""
    import csv
    import glob
    vals = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter and match in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]))
    return vals


def traffic_summary(d):
    """HBM bytes per decode-attention launch from four rocprofv3 --pmc runs
    (FETCH_SIZE and WRITE_SIZE, KiB per dispatch, for `--only decode_attn`
    and for `--only copy`).  Each counter is scaled by bytes / counter of the
    1 GiB copy (it reads 1 GiB and writes 1 GiB).  Prints a markdown summary
    whose `traffic-record:` line bench.py reads back."""
    import statistics
    gib = float(1 << 30)
    cf = _counter_rows(os.path.join(d, "copy_fetch"), "FETCH_SIZE", "copy")
    cw = _counter_rows(os.path.join(d, "copy_write"), "WRITE_SIZE", "copy")
    af = _counter_rows(os.path.join(d, "attn_fetch"), "FETCH_SIZE", "k_decode")
    aw = _counter_rows(os.path.join(d, "attn_write"), "WRITE_SIZE", "k_decode")
    if not (cf and cw and af and aw):
        raise SystemExit(f"missing counter rows under {d}: {len(cf)} {len(cw)} {len(af)} {len(aw)}")
    f_scale = gib / (max(cf) * 1024.0)      # the largest copy dispatch is the 1 GiB one
    w_scale = gib / (max(cw) * 1024.0)
    fetch = statistics.median(af) * 1024.0 * f_scale
    write = statistics.median(aw) * 1024.0 * w_scale
    rec = {"kernel": "decode_attn", "hbm_bytes_per_launch": round(fetch + write),
           "fetch_bytes": round(fetch), "write_bytes": round(write),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "dispatches": [len(af), len(aw)], "source_sha256": kernel_source_hash()}
    print("| quantity | value |\n|---|---|")
    print(f"| FETCH_SIZE, decode attention (KiB/dispatch, median of {len(af)}) | {statistics.median(af):.0f} |")
    print(f"| WRITE_SIZE, decode attention (KiB/dispatch, median of {len(aw)}) | {statistics.median(aw):.0f} |")
    print(f"| FETCH_SIZE, 1 GiB copy (KiB) | {max(cf):.0f} |")
    print(f"| WRITE_SIZE, 1 GiB copy (KiB) | {max(cw):.0f} |")
    print(f"| fetch scale (bytes per counted byte) | {f_scale:.4f} |")
    print(f"| write scale | {w_scale:.4f} |")
    print(f"| HBM bytes per decode-attention launch | {fetch + write:.4g} |")
    print()
    print("traffic-record: " + json.dumps(rec))


def mfma_summary(d, M=8192, N=14336, K=4096, simds=1024, xcds=8, timed=50):
    """MFMA utilisation of the prefill GEMM (k_gemm_big) per dispatch from one
    rocprofv3 --pmc run: busy = SQ_VALU_MFMA_BUSY_CYCLES summed over the
    SIMDs, over GRBM_GUI_ACTIVE x SIMDs (GRBM_GUI_ACTIVE is reported summed
    over the XCDs, so it is divided by their count); the MFMA work checked
    against 2MNK (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts units of 512 FLOPs);
    and the clock the dispatch ran at (GUI-active cycles per XCD over its
    duration)."""
    import csv
    import glob
    import statistics
    rows = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if "k_gemm_big" in r["Kernel_Name"]:
                    key = (f, r["Dispatch_Id"])
                    e = rows.setdefault(key, {"ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                    e[r["Counter_Name"]] = float(r["Counter_Value"])
    need = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")
    rows = [e for e in rows.values() if all(k in e for k in need)]
    if not rows:
        raise SystemExit(f"no k_gemm_big counter rows under {d}")
    util = [e["SQ_VALU_MFMA_BUSY_CYCLES"] / (e["GRBM_GUI_ACTIVE"] / xcds * simds) for e in rows]
    flops = [e["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 for e in rows]
    ghz = [e["GRBM_GUI_ACTIVE"] / xcds / e["ns"] for e in rows]
    us = [e["ns"] / 1e3 for e in rows]
    alg = 2.0 * M * N * K
    med = statistics.median
    print("| quantity (median over %d dispatches, M %d N %d K %d) | value |" % (len(rows), M, N, K))
    print("|---|---|")
    print(f"| MFMA busy / GUI-active cycles (all SIMDs) | {100 * med(util):.1f}% (range {100 * min(util):.1f}-{100 * max(util):.1f}%) |")
    print(f"| MFMA FLOPs counted / 2MNK | {med(flops) / alg:.4f} |")
    print(f"| clock while active (GHz) | {med(ghz):.2f} (range {min(ghz):.2f}-{max(ghz):.2f}) |")
    print(f"| dispatch duration (us) | {med(us):.1f} (range {min(us):.1f}-{max(us):.1f}) |")
    print(f"| achieved / bf16 dense peak at 2.4 GHz (2.5 PFLOP/s) | {100 * alg / (med(us) * 1e-6) / 2.5e15:.1f}% |")
    rec = {"kernel": "k_gemm_big", "M": M, "N": N, "K": K, "dispatches": len(rows),
           "mfma_busy": round(med(util), 4), "mfma_busy_range": [round(min(util), 4), round(max(util), 4)],
           "clock_ghz": round(med(ghz), 3), "flops_counted_over_2mnk": round(med(flops) / alg, 4),
           "source_sha256": kernel_source_hash(MFMA_SOURCES)}
    print()
    print("mfma-record: " + json.dumps(rec))
    # the kernel trace of the same command, when it is under d too: every
    # launch in issue order, and the timed window (the launches after the
    # warm-up) on its own
    tr = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            tr += [(int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                   for r in csv.DictReader(fh) if "k_gemm_big" in r["Kernel_Name"]]
    if tr:
        tr = [x for _, x in sorted(tr)]
        win = tr[-timed:]
        pct = lambda x: 100 * alg / (x * 1e-6) / 2.5e15
        print()
        print(f"Kernel trace: {len(tr)} launches, average {statistics.mean(tr):.1f} us "
              f"({pct(statistics.mean(tr)):.1f}% of peak), min {min(tr):.1f}, max {max(tr):.1f}; "
              f"first 10 launches {statistics.mean(tr[:10]):.1f} us; the last {len(win)} (the timed "
              f"window) {statistics.mean(win):.1f} us ({pct(statistics.mean(win)):.1f}%)")


GEMM_NAMES = ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down")
GEMM_PROFILE = os.path.join(ROOT, "profiles", "decode_gemms_counters_llama3_8b_b64.md")
GEMM_PASSES = {
    "fetch": ("FETCH_SIZE",),
    "write": ("WRITE_SIZE",),
    "tcp": ("TCP_TCC_READ_REQ_sum", "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_PENDING_STALL_CYCLES_sum",
            "TCP_TCR_TCP_STALL_CYCLES_sum", "GRBM_GUI_ACTIVE"),
    "tcc": ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_TAG_STALL_sum", "TCC_REQ_sum", "TA_BUSY_avr",
            "TA_ADDR_STALLED_BY_TC_CYCLES_sum", "GRBM_GUI_ACTIVE"),
    "sq": ("SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY",
           "SQ_BUSY_CYCLES", "SQ_INSTS_VMEM_RD", "SQ_INST_LEVEL_VMEM", "SQ_WAVE_CYCLES",
           "GRBM_GUI_ACTIVE"),
    "tlb": ("TCP_UTCL1_TRANSLATION_MISS_sum", "TCP_UTCL1_TRANSLATION_HIT_sum",
            "TCP_READ_TAGCONFLICT_STALL_CYCLES_sum", "TCP_TOTAL_CACHE_ACCESSES_sum"),
}


def _dispatch_rows(d, match):
    """{dispatch id: {counter: value, 'ns': duration}} of the kernels whose
    name contains `match`, from the rocprofv3 csv output under d."""
    import csv
    import glob
    rows = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if match in r["Kernel_Name"]:
                    e = rows.setdefault(int(r["Dispatch_Id"]), {
                        "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
                    e[r["Counter_Name"]] = float(r["Counter_Value"])
    return rows


def gemm_counters_summary(d, names=GEMM_NAMES, launches=32, warm=3, cus=256, xcds=8):
    """Counters of the decode projection GEMMs at batch 64 from one
    rocprofv3 --pmc pass per subdirectory of d (GEMM_PASSES; each a run of
    `bench.py --only gemm_qkv,gemm_o,gemm_gate_up,gemm_down --launches N`),
    plus copy_fetch / copy_write (the 1 GiB copy that scales FETCH_SIZE and
    WRITE_SIZE) under d or beside it.  The k_gemm_small dispatches of a run come in the order of
    `names`, warm + launches each; the warm-ups are dropped and each counter
    is the median over the timed launches.  Prints a markdown summary whose
    `gemm-counters-record:` line bench.py reads back."""
    import statistics
    med = statistics.median
    per = {n: {} for n in names}
    for pas, counters in GEMM_PASSES.items():
        rows = _dispatch_rows(os.path.join(d, pas), "k_gemm_small")
        ids = sorted(rows)
        if len(ids) != len(names) * (warm + launches):
            raise SystemExit(f"pass {pas}: {len(ids)} k_gemm_small dispatches, expected "
                             f"{len(names) * (warm + launches)}")
        for i, n in enumerate(names):
            block = [rows[k] for k in ids[i * (warm + launches) + warm:(i + 1) * (warm + launches)]]
            for c in counters + ("ns",):
                vals = [e[c] for e in block if c in e]
                if vals:
                    per[n][f"{pas}:{c}"] = med(vals)
    gib = float(1 << 30)
    cd = d if os.path.isdir(os.path.join(d, "copy_fetch")) else os.path.dirname(d.rstrip("/"))
    cf = _counter_rows(os.path.join(cd, "copy_fetch"), "FETCH_SIZE", "copy")
    cw = _counter_rows(os.path.join(cd, "copy_write"), "WRITE_SIZE", "copy")
    f_scale, w_scale = gib / (max(cf) * 1024.0), gib / (max(cw) * 1024.0)
    cfg_b = 64
    shapes = {"gemm_qkv": (6144, 4096), "gemm_o": (4096, 4096), "gemm_gate_up": (28672, 4096),
              "gemm_down": (4096, 14336)}
    recs = {}
    print("| quantity (median over %d launches, batch %d, weights of 32 layers in rotation) | "
          % (launches, cfg_b) + " | ".join(names) + " |")
    print("|---|" + "---|" * len(names))
    table = []
    for n in names:
        e = per[n]
        N, K = shapes[n]
        alg = 2 * N * K + 2 * cfg_b * K + 2 * cfg_b * N
        us = e["tcp:ns"] / 1e3
        hbm = e["fetch:FETCH_SIZE"] * 1024 * f_scale + e["write:WRITE_SIZE"] * 1024 * w_scale
        req = e["tcp:TCP_TCC_READ_REQ_sum"]
        lat = e["tcp:TCP_TCC_READ_REQ_LATENCY_sum"] / max(req, 1.0)
        clk = e["tcp:GRBM_GUI_ACTIVE"] / xcds / e["tcp:ns"]            # GHz
        cyc = e["tcp:GRBM_GUI_ACTIVE"] / xcds
        l2_bytes = req * 128.0                                      # whole 128-byte lines
        per_cu = l2_bytes / cus / (us * 1e-6) / 1e9                 # GB/s into one CU
        inflight = per_cu * 1e9 * (lat / (clk * 1e9)) / 1024.0      # KiB, Little's law
        hit = e["tcc:TCC_HIT_sum"] / max(e["tcc:TCC_HIT_sum"] + e["tcc:TCC_MISS_sum"], 1.0)
        rec = {"us": round(us, 2), "alg_bytes": alg, "hbm_bytes": round(hbm),
               "hbm_over_alg": round(hbm / alg, 3), "hbm_TBps": round(hbm / us / 1e6, 2),
               "l2_to_cu_bytes": round(l2_bytes), "l2_to_cu_over_alg": round(l2_bytes / alg, 2),
               "per_cu_GBps": round(per_cu, 1), "tcp_tcc_read_latency_cycles": round(lat),
               "inflight_KiB_per_cu": round(inflight, 1), "l2_hit": round(hit, 3),
               "clock_ghz": round(clk, 2),
               "tcp_pending_stall_frac": round(e["tcp:TCP_PENDING_STALL_CYCLES_sum"] / cus / cyc, 3),
               "ta_busy_frac": round(e["tcc:TA_BUSY_avr"] / cyc, 3),
               "lds_bank_conflict_per_lds_inst": round(
                   e["sq:SQ_LDS_BANK_CONFLICT"] / max(e["sq:SQ_INSTS_LDS"], 1.0), 3),
               "utcl1_miss": round(e["tlb:TCP_UTCL1_TRANSLATION_MISS_sum"]),
               "utcl1_hit": round(e["tlb:TCP_UTCL1_TRANSLATION_HIT_sum"])}
        recs[n] = rec
    rows_out = [
        ("duration (us)", "us"), ("HBM bytes (FETCH x %.3f + WRITE x %.3f)" % (f_scale, w_scale), "hbm_bytes"),
        ("HBM bytes / algorithmic", "hbm_over_alg"), ("HBM TB/s", "hbm_TBps"),
        ("L2 -> CU bytes (TCP_TCC_READ_REQ x 128)", "l2_to_cu_bytes"),
        ("L2 -> CU bytes / algorithmic", "l2_to_cu_over_alg"), ("intake per CU (GB/s)", "per_cu_GBps"),
        ("mean TCP -> TCC read latency (cycles)", "tcp_tcc_read_latency_cycles"),
        ("bytes in flight per CU, Little's law (KiB)", "inflight_KiB_per_cu"),
        ("L2 hit rate", "l2_hit"), ("clock while active (GHz)", "clock_ghz"),
        ("TCP pending-stall cycles / CU cycles", "tcp_pending_stall_frac"),
        ("TA busy / cycles", "ta_busy_frac"),
        ("LDS bank conflicts per LDS instruction", "lds_bank_conflict_per_lds_inst"),
        ("UTCL1 translation misses", "utcl1_miss"), ("UTCL1 translation hits", "utcl1_hit")]
    for label, key in rows_out:
        print(f"| {label} | " + " | ".join(str(recs[n][key]) for n in names) + " |")
    out = {"kernels": recs, "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "source_sha256": kernel_source_hash(MFMA_SOURCES)}
    print()
    print("gemm-counters-record: " + json.dumps(out))


def measured_gemm_counters():
    """The decode GEMMs' counter record from the committed summary, or None
    when the GEMM sources changed since it was taken."""
    try:
        with open(GEMM_PROFILE) as f:
            lines = [ln for ln in f if ln.startswith("gemm-counters-record: ")]
    except OSError:
        return None
    if not lines:
        return None
    rec = json.loads(lines[-1][len("gemm-counters-record: "):])
    if rec.get("source_sha256") != kernel_source_hash(MFMA_SOURCES):
        return None
    return rec["kernels"]


def measured_mfma():
    """The prefill GEMM's counter record (MFMA busy fraction, clock) from the
    committed summary, or None when its sources changed since."""
    try:
        with open(MFMA_PROFILE) as f:
            lines = [ln for ln in f if ln.startswith("mfma-record: ")]
    except OSError:
        return None
    if not lines:
        return None
    rec = json.loads(lines[-1][len("mfma-record: "):])
    if rec.get("source_sha256") != kernel_source_hash(MFMA_SOURCES):
        return None
    return {k: rec[k] for k in ("mfma_busy", "mfma_busy_range", "clock_ghz",
                                "flops_counted_over_2mnk")}


def measured_traffic():
    """HBM bytes per decode-attention launch from the committed counter
    summary, or None when the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            lines = [ln for ln in f if ln.startswith("traffic-record: ")]
    except OSError:
        return None
    if not lines:
        return None
    rec = json.loads(lines[-1][len("traffic-record: "):])
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec


GEMM_NAMES = ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down")


def decode_attn_long(args, torch, dev, batch=None, parts=None):
    """The paged decode-attention workload on its own: --batch requests with
    KV lengths log-uniform in 128..32768 (seeded), h 32 / h_kv 8 / d_h 128,
    bf16 K and V N(0, 1) in 16-token pages scattered over a pool 1.25x the
    live pages, 256-key chunks.  Two such pools are used in turn, so every
    call reads K and V that are cold in L2 and in the 256 MB last-level
    cache.  Returns (launch, algorithmic bytes, label); with `parts` (a
    dict) it also leaves the first pool's tensors there."""
    import synth
    from invariant_bi_rmsnorm_amd import _lib as L
    B, h, h_kv, d_h, C, ps = batch or args.batch, 32, 8, 128, 256, 16
    kv_len = synth.log_uniform_lengths(B, 128, 32768, seed=args.seed + 31)
    place = synth.scatter_pages(kv_len, ps, seed=args.seed + 32)
    g = torch.Generator(device=dev).manual_seed(args.seed + 33)
    shape = (place.num_pages, h_kv, ps, d_h)
    pools = [tuple(torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(generator=g)
                   for _ in range(2)) for _ in range(2)]
    q = torch.empty((B, h, d_h), dtype=torch.bfloat16, device=dev).normal_(generator=g)
    off = L.bi_chunk_offsets(kv_len, C)
    tot = int(off[-1])
    ml = torch.empty((tot, h, 2), device=dev)
    acc = torch.empty((tot, h, d_h), device=dev)
    bt = torch.from_numpy(place.block_table.copy()).to(dev)
    kvl, offd = torch.from_numpy(kv_len).to(dev), off.to(dev)
    scale = float(1.0 / math.sqrt(d_h))
    turn = [0]

    def fn():
        kp, vp = pools[turn[0] % 2]
        turn[0] += 1
        L.bi_decode_attn(q, kp, vp, bt, kvl, offd, tot, C, scale, ml, acc)

    alg = int(kv_len.sum()) * h_kv * d_h * 2 * 2 + B * h * d_h * 2 + tot * h * (d_h + 2) * 4
    label = (f"decode_attn, batch {B}, KV lengths log-uniform 128..32768 ({int(kv_len.sum())} "
             f"tokens, {tot} chunk rows), two pools in turn")
    if parts is not None:
        parts.update(q=q, k=pools[0][0], v=pools[0][1], block_table=place.block_table,
                     kv_len=kv_len, h_kv=h_kv, chunk=C, scale=scale)
    return fn, alg, label


def prefill_attn_bench(args, torch, dev):
    """Causal prefill attention of one prompt of --prompt tokens (default
    2048) at h 32 / h_kv 8 / d_h 128, 256-key chunks at absolute positions,
    bf16 K and V N(0, 1) already in 16-token pages scattered over a pool (as
    after the prompt's KV append), q N(0, 1).  Algorithmic work: 4 d_h h
    (t + 1) FLOPs for the row at position t (q K^T and P V over its visible
    keys), summed over the prompt; bound: bf16 matrix cores.  Returns
    (launch, FLOPs, label)."""
    import synth
    from invariant_bi_rmsnorm_amd import _lib as L
    T, h, h_kv, d_h, C, ps = args.prompt, 32, 8, 128, 256, 16
    lens = np.array([T], np.int32)
    place = synth.scatter_pages(lens, ps, seed=args.seed + 41)
    g = torch.Generator(device=dev).manual_seed(args.seed + 42)
    shape = (place.num_pages, h_kv, ps, d_h)
    kp = torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(generator=g)
    vp = torch.empty(shape, dtype=torch.bfloat16, device=dev).normal_(generator=g)
    q = torch.empty((T, h, d_h), dtype=torch.bfloat16, device=dev).normal_(generator=g)
    out = torch.empty_like(q)
    qs = torch.tensor([0, T], dtype=torch.int32, device=dev)
    p0 = torch.tensor([0], dtype=torch.int32, device=dev)
    bt = torch.from_numpy(place.block_table.copy()).to(dev)
    scale = float(1.0 / math.sqrt(d_h))

    def fn():
        L.bi_prefill_attn(q, qs, p0, kp, vp, bt, C, scale, out)

    fn.parts = {"q": q, "k": kp, "v": vp, "block_table": place.block_table, "scale": scale}
    flops = 4 * d_h * h * (T * (T + 1) // 2)
    return fn, flops, f"prefill_attn, one prompt of {T} tokens, h 32 / h_kv 8 / d_h 128, chunk {C}"


def _b2b_us(fn, torch, launches=20):
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(launches):
        fn()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / launches


def oracle_table(args, torch, dev):
    """The CPU oracle timed beside the GPU kernels on the workloads the
    scope table names: decode attention with KV lengths log-uniform
    128..32768 at batch 1 and 64, the mixed-batch GEMM at M = 513 (N 14336,
    K 4096), and causal prefill attention of a 2048-token prompt.  Each
    oracle call runs once, on the same inputs as the GPU kernel (K converted
    to the oracle's token-major pages).  Prints one JSON line per
    workload."""
    import oracle
    from invariant_bi_rmsnorm_amd import _lib as L
    threads = oracle.num_threads()

    def line(name, gpu_us, oracle_s, sample):
        print(json.dumps({"oracle_table": name, "gpu_us": round(gpu_us, 2),
                          "oracle_s": round(oracle_s, 3), "oracle_threads": threads,
                          "oracle_over_gpu": round(oracle_s * 1e6 / gpu_us, 1),
                          "sample": sample}), flush=True)

    for B in (1, 64):
        parts = {}
        fn, _, label = decode_attn_long(args, torch, dev, batch=B, parts=parts)
        us = _b2b_us(fn, torch)
        q = parts["q"].float().cpu().numpy()
        kp = L.k_pool_to_rows(parts["k"]).float().cpu().numpy()
        vp = parts["v"].float().cpu().numpy()
        t0 = time.perf_counter()
        oracle.decode_attn(q, kp, vp, parts["block_table"], parts["kv_len"], parts["h_kv"], 16,
                           parts["chunk"], parts["scale"], round_bf16=True, p_bf16=True)
        line(label, us, time.perf_counter() - t0, "the whole call")
        del parts, kp, vp
    M, N, K = 513, 14336, 4096
    g = torch.Generator(device=dev).manual_seed(args.seed + 51)
    A = torch.empty((M, K), dtype=torch.bfloat16, device=dev).normal_(generator=g)
    W = torch.empty((N, K), dtype=torch.bfloat16, device=dev).normal_(0, 0.02, generator=g)
    Cm = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    Wp = L.pack_weight(W)
    us = _b2b_us(lambda: L.bi_gemm(A, Wp, Cm), torch)
    Ac, Wc = A.float().cpu().numpy(), W.float().cpu().numpy()
    t0 = time.perf_counter()
    oracle.gemm(Ac, Wc, True)
    line(f"bi_gemm M {M} N {N} K {K} (bf16 in and out)", us, time.perf_counter() - t0,
         "the whole product")
    del A, W, Cm, Ac, Wc
    fn, _, label = prefill_attn_bench(args, torch, dev)
    us = _b2b_us(fn, torch)
    T, parts = args.prompt, fn.parts
    q = parts["q"].float().cpu().numpy()
    kp = L.k_pool_to_rows(parts["k"]).float().cpu().numpy()
    vp = parts["v"].float().cpu().numpy()
    t0 = time.perf_counter()
    oracle.prefill_attn(q, np.array([0, T], np.int32), np.array([0], np.int32), kp, vp,
                        parts["block_table"], 8, 16, 256, parts["scale"], round_bf16=True,
                        p_bf16=True)
    line(label, us, time.perf_counter() - t0, "the whole prompt")


def only_gemms(args, torch, dev, names):
    """The decode step's projection GEMMs at the bench's batch, each launched
    --launches times back to back, cycling through the weights of all the
    model's layers as the step does (each launch reads weights that are cold
    in L2 and in the 256 MB last-level cache), in the order given.  The
    activations are N(0, 1); the QKV product runs with its RoPE + KV-append
    epilogue and the gate/up product with its SwiGLU epilogue, as in the
    step.  Prints one JSON line per GEMM."""
    from invariant_bi_rmsnorm_amd import _lib as L
    from invariant_bi_rmsnorm_amd.model import init_weights
    cfg = model_config(args)
    w = init_weights(cfg, args.seed + 14, dev, source="device")
    _, eng, _, meta, kv_len, _, _ = build_workload(args, args.batch, torch, dev, w)
    T = meta["T"]
    c = cfg
    for buf in (eng.x, eng.att, eng.act):
        buf.normal_()
    nl = len(w.layers)

    def fn_for(name, i):
        lw = eng.w.layers[i % nl]   # the engine's packed weights
        if name == "gemm_qkv":
            return lambda: L.bi_gemm_qkv_rope(
                eng.x[:T], lw.wqkv, c.h, c.h_kv, c.d_h, meta["pos"], eng.cos, eng.sin,
                meta["slots"], eng.q[:T], eng.pool.k[i % nl], eng.pool.v[i % nl])
        if name == "gemm_o":
            return lambda: L.bi_gemm(eng.att[:T].view(T, c.h * c.d_h), lw.wo, eng.o[:T])
        if name == "gemm_gate_up":
            return lambda: L.bi_gemm_swiglu(eng.x[:T], lw.wgu, eng.act[:T])
        return lambda: L.bi_gemm(eng.act[:T], lw.wdown, eng.o[:T])

    for name in names:
        fns = [fn_for(name, i) for i in range(nl)]
        for f in fns[:3]:
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.launches):
            fns[i % nl]()
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / args.launches
        alg = algorithmic_bytes(name, cfg, args.batch, kv_len, meta)
        print(json.dumps({"kernel": f"{name}, batch {args.batch}", "launches": args.launches,
                          "warmup_launches": 3, "weights": f"{nl} layers in rotation",
                          "avg_us": round(us, 2), "alg_bytes": alg,
                          "GBps": round(alg / us / 1e3, 1),
                          "hbm_frac": round(alg / us / 1e3 / (HBM_PEAK / 1e9), 4)}), flush=True)


def only_kernel(args, torch, dev):
    """Launch one kernel of the step (the last layer's instance) --launches
    times back to back and report its average duration from HIP events on
    its stream.  'copy' copies 1 GiB device to device (the yardstick that
    calibrates HBM byte counters)."""
    names = [n for n in args.only.split(",") if n]
    if names and all(n in GEMM_NAMES for n in names):
        only_gemms(args, torch, dev, names)
        return
    if args.only == "copy":
        n = 1 << 28
        src = torch.empty(n, device=dev).normal_()
        dst = torch.empty_like(src)
        fn, alg, label = (lambda: dst.copy_(src)), 2 * 4 * n, "copy 1 GiB"
    elif args.only == "prefill_gemm":
        print(json.dumps(prefill_gemm(torch, dev, launches=args.launches)), flush=True)
        return
    elif args.only == "decode_attn_long":
        fn, alg, label = decode_attn_long(args, torch, dev)
    elif args.only == "prefill_attn":
        fn, flops, label = prefill_attn_bench(args, torch, dev)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.launches):
            fn()
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / args.launches
        tf = flops / us / 1e6
        print(json.dumps({"kernel": label, "launches": args.launches, "avg_us": round(us, 2),
                          "flops": flops, "TFLOPs": round(tf, 1), "bound": "mfma",
                          "peak_TFLOPs": BF16_PEAK / 1e12,
                          "frac": round(tf * 1e12 / BF16_PEAK, 4)}), flush=True)
        return
    elif args.only == "log_softmax":
        # logprobs of a decode batch: fp32 logits [batch, vocab], read once and
        # written once (the second and third passes over a row hit L2)
        from invariant_bi_rmsnorm_amd import _lib
        V = model_config(args).vocab
        x = torch.empty((args.batch, V), device=dev).normal_(std=3.0)
        y = torch.empty_like(x)
        fn, alg = (lambda: _lib.bi_log_softmax(x, y)), 2 * 4 * args.batch * V
        label = f"log_softmax, batch {args.batch}"
    elif args.only == "sample":
        # seeded Gumbel-max draw per row over fp32 logits [batch, vocab]
        from invariant_bi_rmsnorm_amd import _lib
        V = model_config(args).vocab
        x = torch.empty((args.batch, V), device=dev).normal_(std=3.0)
        sd = torch.arange(args.batch, dtype=torch.int32, device=dev)
        ps = torch.full((args.batch,), 1000, dtype=torch.int32, device=dev)
        tp = torch.full((args.batch,), 0.8, dtype=torch.float32, device=dev)
        out = torch.empty(args.batch, dtype=torch.int32, device=dev)
        fn, alg = (lambda: _lib.bi_sample(x, sd, ps, tp, out)), 4 * args.batch * V
        label = f"sample, batch {args.batch}"
    else:
        from invariant_bi_rmsnorm_amd.model import init_weights
        cfg = model_config(args)
        w = init_weights(cfg, args.seed + 14, dev, source="device")
        _, eng, twin, meta, kv_len, _, tmeta = build_workload(
            args, args.batch, torch, dev, w, free=args.twin,
            twin_mode=args.twin_mode)
        e, meta = (twin, tmeta) if args.twin else (eng, meta)
        grab = {}

        def keep(name, f):
            grab[name] = f
            f()

        e.forward(meta, timer=keep)
        torch.cuda.synchronize()
        if args.only not in grab:
            raise SystemExit(f"--only {args.only}: not a kernel of the step ({sorted(grab)})")
        fn = grab[args.only]
        if args.only == "decode_attn" and not args.twin:   # the partial kernel alone
            fn = e.decode_partials_launch(meta, cfg.layers - 1)
        alg = algorithmic_bytes(args.only, cfg, args.batch, kv_len, meta)
        label = f"{args.only}{' (twin)' if args.twin else ''}, batch {args.batch}"
        if args.only == "decode_attn" and not args.twin:
            label += " (bi_decode_attn alone, without the merge)"
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.launches):
        fn()
    b.record()
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / args.launches
    out = {"kernel": label, "launches": args.launches, "avg_us": round(us, 2)}
    if alg:
        out.update(alg_bytes=alg, GBps=round(alg / us / 1e3, 1),
                   hbm_frac=round(alg / us / 1e3 / (HBM_PEAK / 1e9), 4))
    print(json.dumps(out), flush=True)


def dvr_compare(args, torch, dev):
    """Decode-verify-rollback ("LLM-42", "The Decode-Verify-Rollback
    Protocol") with the twins as the fast path and the invariant kernels as
    the verifier, against greedy decoding on the invariant kernels alone and
    on the twins alone: the same prompts, eager steps for all three (host
    launch time included alike), tokens per second over the generated tokens
    after the prompts' prefill."""
    import synth
    from invariant_bi_rmsnorm_amd import harness as H
    from invariant_bi_rmsnorm_amd.model import Engine, KVPool, init_weights
    cfg = model_config(args)
    B, new, win, grp = args.batch if args.batch != 64 else 8, args.dvr_new, args.dvr_window, \
        args.dvr_group
    w = init_weights(cfg, args.seed + 14, dev, source="device")
    lens = synth.uniform_lengths(B, 256, 1024, seed=args.seed + 21)
    prompts = [[int(t) for t in synth.token_ids(int(n), cfg.vocab, seed=args.seed + 100 + r)]
               for r, n in enumerate(lens)]
    per = (int(lens.max()) + new + win + cfg.page_size) // cfg.page_size + 1
    pool = KVPool(cfg, B * per, dev)
    pages = [list(range(r * per, (r + 1) * per)) for r in range(B)]
    chunk = 512
    rows = max(B * chunk, grp * win, B)
    inv = Engine(cfg, w, pool, dev, max_rows=rows, max_pages_per_req=per)
    fast = Engine(cfg, w, pool, dev, max_rows=rows, max_pages_per_req=per, free=True)

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = fn()
        torch.cuda.synchronize()
        return out, time.perf_counter() - t0

    def prefill_time(engine):
        return timed(lambda: H._prefill(engine, prompts, pages, chunk))[1]

    # warm both engines (kernel attributes, workspaces) on a short run
    H.greedy_decode(inv, prompts, pages, 4, chunk=chunk)
    H.decode_verify_rollback(fast, inv, prompts, pages, 4, window=2, group=grp, chunk=chunk)
    res = {}
    ref, t = timed(lambda: H.greedy_decode(inv, prompts, pages, new, chunk=chunk))
    res["invariant"] = t - prefill_time(inv)
    fast_seq, t = timed(lambda: H.greedy_decode(fast, prompts, pages, new, chunk=chunk))
    res["twins"] = t - prefill_time(fast)
    (dvr_seq, st), t = timed(lambda: H.decode_verify_rollback(fast, inv, prompts, pages, new,
                                                              window=win, group=grp,
                                                              chunk=chunk))
    res["dvr"] = t - prefill_time(inv)
    toks = B * (new - 1)
    line = {
        "mode": "decode-verify-rollback", "batch": B, "prompt_lens": [int(v) for v in lens],
        "new_tokens": new, "window": win, "verify_group": grp, "steps": "eager",
        "tokens_per_s": {k: round(toks / v, 1) for k, v in res.items()},
        "dvr_vs_invariant_pct": round(100.0 * (res["dvr"] / res["invariant"] - 1.0), 1),
        "dvr_equals_invariant_greedy": dvr_seq == ref,
        "twins_equal_invariant_greedy": fast_seq == ref,
        "windows": st.windows, "mismatched_windows": st.mismatches,
        "discarded_candidates": st.discarded, "fast_steps": st.fast_steps,
        "verify_launches": st.verify_steps,
    }
    print(json.dumps(line), flush=True)


def _rounded(d):
    return {k: (round(v, 3) if isinstance(v, float) else v) for k, v in d.items()}


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(args.traffic_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary, timed=args.launches)
        return
    if args.gemm_counters_summary:
        gemm_counters_summary(args.gemm_counters_summary, launches=args.launches)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path is "
              "data-parallel across GPUs and nothing here uses a second device", file=sys.stderr)
        sys.exit(2)
    import torch
    from invariant_bi_rmsnorm_amd import _lib
    from invariant_bi_rmsnorm_amd.model import init_weights
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    _lib.load()
    dev = torch.device("cuda:0")
    if args.oracle_table:
        oracle_table(args, torch, dev)
        return
    if args.only:
        only_kernel(args, torch, dev)
        return
    if args.dvr:
        dvr_compare(args, torch, dev)
        return
    cfg = model_config(args)
    w = init_weights(cfg, args.seed + 14, dev, source="device")
    log(f"weights drawn ({cfg.weight_bytes() / 1e9:.2f} GB)")
    B = args.batch
    res, detail = run_batch(args, B, torch, dev, w, want_detail=True)
    per, per_free = detail["per_kernel"], detail["per_kernel_free"]
    kv_len, meta = detail["kv_len"], detail["meta"]
    for name in per:
        b = algorithmic_bytes(name, cfg, B, kv_len, meta)
        if b is not None:
            per[name]["alg_bytes"] = b
            per[name]["GBps"] = b / (per[name]["avg_us"] * 1e-6) / 1e9
            per[name]["hbm_frac"] = per[name]["GBps"] * 1e9 / HBM_PEAK
    dom = max((n for n in per if "alg_bytes" in per[n]),
              key=lambda n: per[n]["total_ms_per_step"])
    b = per[dom]["alg_bytes"]
    if dom == "decode_attn":   # the partial kernel alone: the merge is its own kernel
        fn = detail["eng"].decode_partials_launch(meta, cfg.layers - 1)
        timing = ("20 back-to-back launches of bi_decode_attn (the step's last-layer "
                  "instance, without the merge) between one HIP event pair on its stream")
    else:
        fn = detail["grab"][dom]
        timing = ("20 back-to-back launches of the step's last-layer instance between one "
                  "HIP event pair on its stream")
    us = back_to_back_us(fn, torch)
    achieved = b / (us * 1e-6) / 1e9
    rl = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK / 1e9,
          "unit": "GB/s", "frac": round(achieved * 1e9 / HBM_PEAK, 4), "traffic": None,
          "avg_launch_us": round(us, 2), "alg_bytes_per_launch": b, "timing": timing,
          "avg_launch_us_event_pairs": round(per[dom]["avg_us"], 2),
          "event_pairs_note": "per-launch event pairs bracket the whole call site "
                              "(for decode_attn: partials and merge)"}
    rec = measured_traffic() if dom == "decode_attn" else None
    if rec is not None:
        rl["traffic"] = rec["hbm_bytes_per_launch"]
        rl["traffic_frac_of_alg"] = round(rec["hbm_bytes_per_launch"] / b, 4)
    out = {
        "metric": METRIC, "value": round(res["inv"]["tokens_per_s"], 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(res["inv"]["ms_per_step"], 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped decode step, 32 layers, batch 64, "
                               "KV lengths uniform 32-4096, kv chunk 256, 16-token pages",
                   "layers": cfg.layers, "global_batch": B, "kv_tokens": int(sum(kv_len)),
                   "parallelism": "none (1 GPU)"},
        "roofline": rl,
        "step_hbm_frac": round(res["hbm_frac_of_step_bound"], 4),
        "invariance_overhead_pct": round(res["invariance_overhead_pct"], 2),
        "twin_tokens_per_s": round(res["free"]["tokens_per_s"], 1),
        "twin": {"mode": "tuned: per call site, the fastest of the invariant configuration "
                         "and the batch-adaptive ones, measured on first use",
                 "timing": "graph replay" if res["free"]["graph"] else "eager steps",
                 "graph_matches_eager": res["free"]["graph_matches_eager"],
                 "graph_check": "within 1e-3 of the largest logit (its kernels need not "
                                "repeat their bits)",
                 "choices": res["twin_choices"]},
        "graph": res["inv"]["graph"], "graph_matches_eager": res["inv"]["graph_matches_eager"],
        "per_kernel_note": "HIP event pairs around each launch of 20 eager steps, a device "
                           "spin ahead of each start event; each pair adds its own cost of a "
                           "few us, so short kernels read high (profiles/ has their "
                           "kernel-trace durations)",
        "per_kernel": {k: _rounded(v) for k, v in per.items()},
        "per_kernel_twin": {k: _rounded(v) for k, v in per_free.items()},
        "per_kernel_delta_us": {k: round(per[k]["avg_us"] - per_free[k]["avg_us"], 2)
                                for k in per if k in per_free},
    }
    gc = measured_gemm_counters()
    if gc is not None:
        # counter record of the projection GEMMs (profiles/), while their
        # sources match it: HBM and L2 -> CU bytes over the algorithmic ones,
        # the intake per CU and the bytes it keeps in flight
        out["gemm_counters"] = {k: {f: v[f] for f in ("hbm_over_alg", "l2_to_cu_over_alg",
                                                      "per_cu_GBps", "inflight_KiB_per_cu",
                                                      "tcp_pending_stall_frac")}
                                for k, v in gc.items()}
    sweep = [int(x) for x in args.sweep.split(",") if x.strip()]
    if sweep:
        keep = detail
        detail = None
        out["sweep"] = {}
        for b2 in sweep:
            r2, _ = run_batch(args, b2, torch, dev, w, want_detail=False)
            out["sweep"][str(b2)] = {
                "tokens_per_s": round(r2["inv"]["tokens_per_s"], 1),
                "ms_per_step": round(r2["inv"]["ms_per_step"], 3),
                "twin_tokens_per_s": round(r2["free"]["tokens_per_s"], 1),
                "twin_timing": "graph replay" if r2["free"]["graph"] else "eager steps",
                "invariance_overhead_pct": round(r2["invariance_overhead_pct"], 2),
                "twin_choices": {k: v["picked"] for k, v in r2["twin_choices"].items()},
                "step_hbm_frac": round(r2["hbm_frac_of_step_bound"], 4)}
            torch.cuda.empty_cache()
        detail = keep
    out["prefill_gemm"] = prefill_gemm(torch, dev)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(args, detail, B)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
