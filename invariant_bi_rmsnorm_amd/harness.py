"""Schedule fuzzer and bitwise verdict for batch invariance.

"Lockstep", section "Proving it": enumerate and randomise what a scheduler
may vary -- which requests share a batch, arrival order, where preemption
lands, eviction and readmission -- replay a fixed set of prompts under each
schedule and compare logits bit for bit with the single-request baseline;
any difference fails.  The split between a pure diff/verdict core (no GPU,
no engine) and an impure driver follows the verifier described on
"llamacpp-batch-invariance" (pure core vs driver), as do its anti-vacuity
floors: a pass only counts if requests really were co-batched and really
completed, and a clean result carries the rule-of-three bound 3/n.

Driver model.  A request's sequence is prompt + generated tokens; the cache
holds its first `computed` positions.  A step gives each chosen request a
segment of rows [computed, computed + n); a segment that reaches the end of
the sequence yields the next token's logits (greedy: token = argmax).
Preemption frees a request's pages; readmission either swaps the saved KV
bytes back into freshly drawn pages or recomputes the whole sequence by
prefill (in random chunk cuts).  Logits produced again for a position
already recorded must equal the first record.
"""
from __future__ import annotations

import hashlib
import json
import os
import tempfile
from dataclasses import dataclass, field

import numpy as np

GREEN, RED, UNVERIFIED = "GREEN", "RED", "UNVERIFIED"


# ---------------------------------------------------------------------------
# pure core
# ---------------------------------------------------------------------------

def logits_digest(row_bytes: bytes) -> str:
    return hashlib.sha256(row_bytes).hexdigest()[:32]


def diff_runs(baseline: dict, runs: list) -> dict:
    """baseline: {rid: {pos: digest}}; runs: list of {rid: {pos: digest}}.
    Returns per-request divergence counts and the distinct digests seen per
    (request, position) across baseline and runs ("unique samples")."""
    divergent = {}
    unique_max = 1
    compared = 0
    missing = 0
    for rid, ref in baseline.items():
        bad = 0
        for pos, dig in ref.items():
            seen = {dig}
            for run in runs:
                got = run.get(rid, {}).get(pos)
                if got is None:
                    missing += 1
                    continue
                compared += 1
                if got != dig:
                    bad += 1
                seen.add(got)
            unique_max = max(unique_max, len(seen))
        if bad:
            divergent[rid] = bad
    return {"divergent": divergent, "compared": compared, "missing": missing,
            "unique_samples_max": unique_max}


def decide(report: dict, cobatched: dict, completed: dict, n_requests: int,
           min_cobatch_frac: float = 1.0, min_completion_frac: float = 1.0) -> dict:
    """Verdict: RED on any divergence (exact match only -- a tolerance would
    turn a real divergence into a pass); otherwise GREEN only if the run
    earned it (co-batching and completion floors), else UNVERIFIED."""
    cob = sum(1 for v in cobatched.values() if v > 0) / max(1, n_requests)
    comp = sum(1 for v in completed.values() if v) / max(1, n_requests)
    n = report["compared"]
    out = {"compared": n, "divergent_requests": len(report["divergent"]),
           "unique_samples_max": report["unique_samples_max"], "missing": report["missing"],
           "cobatch_frac": cob, "completion_frac": comp,
           "rule_of_three_upper": (3.0 / n) if n else None}
    if report["divergent"]:
        out["verdict"] = RED
    elif cob < min_cobatch_frac or comp < min_completion_frac or n == 0 or report["missing"]:
        out["verdict"] = UNVERIFIED
    else:
        out["verdict"] = GREEN
    return out


def write_report(path: str, report: dict) -> None:
    """Atomic JSON write (temp file + rename): a reader never sees half a file."""
    d = os.path.dirname(os.path.abspath(path))
    os.makedirs(d, exist_ok=True)
    fd, tmp = tempfile.mkstemp(dir=d, suffix=".tmp")
    with os.fdopen(fd, "w") as f:
        json.dump(report, f, indent=1, sort_keys=True)
    os.replace(tmp, path)


# ---------------------------------------------------------------------------
# driver
# ---------------------------------------------------------------------------

@dataclass
class Request:
    rid: int
    prompt: list
    max_new: int
    generated: list = field(default_factory=list)
    pages: list = field(default_factory=list)
    computed: int = 0
    state: str = "waiting"        # waiting | running | preempted | done
    saved_kv: object = None       # swapped-out KV bytes
    records: dict = field(default_factory=dict)
    rerecord_mismatch: int = 0
    cobatched_steps: int = 0

    @property
    def seq(self):
        return self.prompt + self.generated

    def done(self) -> bool:
        return len(self.generated) >= self.max_new


class PagePool:
    def __init__(self, num_pages: int, rng: np.random.Generator):
        self.free = list(range(num_pages))
        self.rng = rng

    def take(self, n: int) -> list:
        if n > len(self.free):
            raise RuntimeError("page pool exhausted")
        idx = self.rng.choice(len(self.free), size=n, replace=False)
        got = [self.free[i] for i in idx]
        for i in sorted(idx, reverse=True):
            self.free.pop(i)
        return got

    def give(self, pages: list) -> None:
        self.free.extend(pages)


@dataclass
class FuzzConfig:
    seed: int = 0
    max_rows: int = 512          # token budget of one step
    max_reqs: int = 64           # segments per step
    p_preempt: float = 0.05      # per step, chance to preempt one running request
    p_swap: float = 0.5          # readmission by swap (else recompute)
    prefill_whole: bool = False  # baseline: prompt in one segment
    alone: bool = False          # baseline: one request at a time
    p_full: float = 0.0          # per step, chance to take every runnable request
    arrival_steps: int | None = None   # arrivals spread over this many steps


class Runner:
    """Runs requests through an engine-like backend under a fuzzed (or the
    baseline) schedule.  Backend interface:
        backend.page_size, backend.num_pages
        backend.step(segments) -> (list of logits-row bytes, list of argmax)
          for the segments with want_logits, in order
        backend.swap_out(pages) -> blob ; backend.swap_in(blob, pages)
    """

    def __init__(self, backend, reqs: list, fz: FuzzConfig):
        self.b, self.fz = backend, fz
        self.rng = np.random.Generator(np.random.PCG64(fz.seed))
        self.pool = PagePool(backend.num_pages, self.rng)
        self.reqs = [Request(r.rid, list(r.prompt), r.max_new) for r in reqs]
        self.steps = 0
        self.max_segments = 0     # most requests in one step
        self.max_rows = 0         # most rows in one step
        self.swaps = 0            # preemptions readmitted by swap
        self.recomputes = 0       # preemptions readmitted by recompute

    def _ensure_pages(self, r: Request, upto: int):
        need = -(-upto // self.b.page_size) - len(r.pages)
        if need > 0:
            r.pages += self.pool.take(need)

    def _preempt(self, r: Request):
        if self.rng.random() < self.fz.p_swap and r.computed > 0:
            r.saved_kv = (self.b.swap_out(r.pages), r.computed)
            self.swaps += 1
        else:
            r.saved_kv = None
            r.computed = 0
            self.recomputes += 1
        self.pool.give(r.pages)
        r.pages = []
        r.state = "preempted"

    def _readmit(self, r: Request):
        if r.saved_kv is not None:
            blob, computed = r.saved_kv
            self._ensure_pages(r, computed)
            self.b.swap_in(blob, r.pages)
            r.computed = computed
            r.saved_kv = None
        r.state = "running"

    def _segment_len(self, r: Request, budget: int) -> int:
        rem = len(r.seq) - r.computed
        if rem == 1 or self.fz.prefill_whole:
            return rem
        cut = int(self.rng.integers(1, rem + 1))
        return max(1, min(cut, budget))

    def run(self) -> dict:
        from .model import Segment
        fz, rng = self.fz, self.rng
        order = list(range(len(self.reqs)))
        if not fz.alone:
            rng.shuffle(order)
        spread = fz.arrival_steps if fz.arrival_steps is not None else 4 + len(order) // 2
        arrivals = {rid: (0 if fz.alone else int(rng.integers(0, max(1, spread))))
                    for rid in order}
        pending = list(order)
        while any(not r.done() for r in self.reqs):
            self.steps += 1
            if self.steps > 100000:
                raise RuntimeError("schedule did not finish")
            # arrivals (alone: the next request only when the previous is done)
            if fz.alone:
                if not any(r.state == "running" for r in self.reqs) and pending:
                    self.reqs[pending.pop(0)].state = "running"
            else:
                for rid in list(pending):
                    if arrivals[rid] <= self.steps:
                        self.reqs[rid].state = "running"
                        pending.remove(rid)
            running = [r for r in self.reqs if r.state == "running" and not r.done()]
            # preemption / readmission
            if not fz.alone and running and rng.random() < fz.p_preempt:
                self._preempt(running[int(rng.integers(len(running)))])
            for r in self.reqs:
                if r.state == "preempted" and rng.random() < 0.5:
                    self._readmit(r)
            runnable = [r for r in self.reqs if r.state == "running" and not r.done()]
            if not runnable:
                continue
            share = None
            if fz.alone:
                chosen = runnable[:1]
            elif fz.p_full > 0 and rng.random() < fz.p_full:
                # every runnable request, each with an equal share of the rows
                perm = rng.permutation(len(runnable))[:fz.max_reqs]
                chosen = [runnable[int(i)] for i in perm]
                share = max(1, fz.max_rows // len(chosen))
            else:
                k = int(rng.integers(1, min(len(runnable), fz.max_reqs) + 1))
                chosen = list(rng.choice(runnable, size=k, replace=False))
            segs, owners, budget = [], [], fz.max_rows
            for r in chosen:
                if budget <= 0:
                    break
                n = self._segment_len(r, budget if share is None else min(share, budget))
                budget -= n
                upto = r.computed + n
                try:
                    self._ensure_pages(r, upto)
                except RuntimeError:
                    self._preempt(r)
                    continue
                want = upto == len(r.seq)
                segs.append(Segment(pages=list(r.pages), pos0=r.computed,
                                    tokens=r.seq[r.computed:upto], want_logits=want))
                owners.append((r, upto, want))
            if not segs:
                continue
            self.max_segments = max(self.max_segments, len(segs))
            self.max_rows = max(self.max_rows, sum(len(sg.tokens) for sg in segs))
            rows, toks = self.b.step(segs)
            it = iter(zip(rows, toks))
            for r, upto, want in owners:
                r.computed = upto
                if len(segs) > 1:
                    r.cobatched_steps += 1
                if want:
                    row, tok = next(it)
                    pos = upto - 1
                    dig = logits_digest(row)
                    if pos in r.records and r.records[pos] != dig:
                        r.rerecord_mismatch += 1
                    r.records.setdefault(pos, dig)
                    if len(r.generated) < r.max_new and upto == len(r.seq):
                        r.generated.append(int(tok))
                    if r.done():
                        r.state = "done"
                        self.pool.give(r.pages)
                        r.pages = []
        return {r.rid: dict(r.records) for r in self.reqs}


def verify(backend_factory, reqs: list, n_schedules: int, fuzz,
           report_path: str | None = None) -> dict:
    """Baseline (each request alone, prompt in one prefill) against fuzzed
    schedules; returns (and optionally writes) the verdict report.  fuzz: a
    FuzzConfig, run under n_schedules seeds derived from its seed, or a list
    of FuzzConfigs, one schedule each (n_schedules is then ignored)."""
    first = fuzz[0] if isinstance(fuzz, (list, tuple)) else fuzz
    base = Runner(backend_factory(), reqs, FuzzConfig(seed=first.seed, alone=True,
                                                      prefill_whole=True)).run()
    runs, cob, comp, remis = [], {r.rid: 0 for r in reqs}, {r.rid: True for r in reqs}, 0
    if isinstance(fuzz, (list, tuple)):
        configs = list(fuzz)
    else:
        seeds = np.random.Generator(np.random.PCG64(fuzz.seed + 1)).integers(1, 2**31,
                                                                             n_schedules)
        configs = [FuzzConfig(**{**fuzz.__dict__, "seed": int(s)}) for s in seeds]
    max_segments = max_rows = swaps = recomputes = 0
    for fz in configs:
        runner = Runner(backend_factory(), reqs, fz)
        runs.append(runner.run())
        max_segments = max(max_segments, runner.max_segments)
        max_rows = max(max_rows, runner.max_rows)
        swaps += runner.swaps
        recomputes += runner.recomputes
        for r in runner.reqs:
            cob[r.rid] += r.cobatched_steps
            comp[r.rid] = comp[r.rid] and r.done()
            remis += r.rerecord_mismatch
    rep = diff_runs(base, runs)
    out = decide(rep, cob, comp, len(reqs))
    out["rerecord_mismatch"] = remis
    if remis:
        out["verdict"] = RED
    out["schedules"] = len(configs)
    out["max_requests_per_step"] = max_segments
    out["max_rows_per_step"] = max_rows
    out["preemptions"] = {"swap": swaps, "recompute": recomputes}
    out["schedule_seeds"] = [int(fz.seed) for fz in configs]
    out["divergent"] = {str(k): v for k, v in rep["divergent"].items()}
    if report_path:
        write_report(report_path, out)
    return out


class EngineBackend:
    """Adapter from model.Engine to the Runner's backend interface."""

    def __init__(self, engine):
        self.e = engine
        self.page_size = engine.cfg.page_size
        self.num_pages = engine.pool.num_pages

    def step(self, segs):
        out = self.e.step(segs)
        if not out.seg_index:
            return [], []
        logits = out.logits.cpu().numpy()
        toks = out.tokens.cpu().numpy()
        # engine returns rows in packed (decode-first) order; map back to
        # the order of the segments that asked for logits
        pos = {si: k for k, si in enumerate(out.seg_index)}
        wanted = [i for i, s in enumerate(segs) if s.want_logits]
        return ([logits[pos[i]].tobytes() for i in wanted], [int(toks[pos[i]]) for i in wanted])

    def swap_out(self, pages):
        idx = self._idx(pages)
        return (self.e.pool.k[:, idx].cpu(), self.e.pool.v[:, idx].cpu())

    def swap_in(self, blob, pages):
        idx = self._idx(pages)
        k, v = blob
        n = k.shape[1]
        self.e.pool.k[:, idx[:n]] = k.to(self.e.pool.k.device)
        self.e.pool.v[:, idx[:n]] = v.to(self.e.pool.v.device)

    def _idx(self, pages):
        import torch
        return torch.tensor(pages, dtype=torch.long, device=self.e.pool.k.device)


# ---------------------------------------------------------------------------
# decode-verify-rollback over the twins
# ---------------------------------------------------------------------------
# "LLM-42: ... verified speculation", "The Decode-Verify-Rollback Protocol":
# decode a window of tokens on the fast, batch-adaptive path; replay the
# window under the fixed reduction schedule in verify batches of a few
# requests; commit the candidates up to the first one the replay disagrees
# with, plus the replay's own token there, and resume decoding from it.  Here
# the fast path is an engine on the twins and the verifier an engine on the
# invariant kernels, over one shared KV pool: the replay is a prefill of the
# window (every row's logits) that also rewrites the window's KV with the
# invariant values, so every committed token equals greedy decoding on the
# invariant kernels alone.

@dataclass
class DvrStats:
    windows: int = 0          # windows verified (per request)
    verify_steps: int = 0     # verifier launches (groups of requests)
    fast_steps: int = 0       # decode steps on the fast path
    committed: int = 0        # tokens committed after verification
    mismatches: int = 0       # windows cut at a disagreeing token
    discarded: int = 0        # fast candidates thrown away by rollbacks


def _prefill(engine, prompts, pages, chunk):
    """Prefill every prompt (chunks of at most `chunk` rows per request);
    returns the argmax token after each prompt."""
    firsts = [None] * len(prompts)
    done = [0] * len(prompts)
    while any(d < len(p) for d, p in zip(done, prompts)):
        segs, who = [], []
        for r, p in enumerate(prompts):
            if done[r] < len(p):
                n = min(chunk, len(p) - done[r])
                segs.append(_seg(pages[r], done[r], p[done[r]:done[r] + n]))
                who.append((r, done[r] + n == len(p)))
                done[r] += n
        out = engine.step(segs)
        toks = out.tokens.cpu().numpy()
        for k, si in enumerate(out.seg_index):
            r, last = who[si]
            if last:
                firsts[r] = int(toks[k])
    return firsts


def _seg(pages, pos0, tokens, all_logits=False):
    from .model import Segment
    return Segment(pages=pages, pos0=pos0, tokens=list(tokens), want_logits=True,
                   all_logits=all_logits)


def greedy_decode(engine, prompts, pages, max_new, chunk=256):
    """Greedy generation on one engine: all live requests decode together."""
    seqs = [[t] for t in _prefill(engine, prompts, pages, chunk)]
    while True:
        live = [r for r in range(len(prompts)) if len(seqs[r]) < max_new]
        if not live:
            return seqs
        segs = [_seg(pages[r], len(prompts[r]) + len(seqs[r]) - 1, [seqs[r][-1]]) for r in live]
        out = engine.step(segs)
        toks = out.tokens.cpu().numpy()
        for k, si in enumerate(out.seg_index):
            seqs[live[si]].append(int(toks[k]))


def decode_verify_rollback(fast, verifier, prompts, pages, max_new, window=64, group=8,
                           chunk=256):
    """Generate max_new tokens per request by decode-verify-rollback.  `fast`
    and `verifier` are engines over the same KV pool; `pages[r]` must hold
    len(prompts[r]) + max_new + window positions.  Returns (tokens, DvrStats)."""
    st = DvrStats()
    seqs = [[t] for t in _prefill(verifier, prompts, pages, chunk)]
    n = len(prompts)
    while True:
        live = [r for r in range(n) if len(seqs[r]) < max_new]
        if not live:
            return seqs, st
        # decode: a window of candidates for every live request, batched
        want = {r: min(window, max_new - len(seqs[r])) for r in live}
        cand = {r: [] for r in live}
        for step in range(max(want.values())):
            act = [r for r in live if len(cand[r]) < want[r]]
            segs = []
            for r in act:
                ctx = seqs[r] + cand[r]
                segs.append(_seg(pages[r], len(prompts[r]) + len(ctx) - 1, [ctx[-1]]))
            out = fast.step(segs)
            st.fast_steps += 1
            toks = out.tokens.cpu().numpy()
            for k, si in enumerate(out.seg_index):
                cand[act[si]].append(int(toks[k]))
        # verify: replay each window (the last committed token, then all but
        # the last candidate) in groups, every row's logits
        for g0 in range(0, len(live), group):
            grp = live[g0:g0 + group]
            segs = [_seg(pages[r], len(prompts[r]) + len(seqs[r]) - 1,
                         [seqs[r][-1]] + cand[r][:-1], all_logits=True) for r in grp]
            out = verifier.step(segs)
            st.verify_steps += 1
            toks = out.tokens.cpu().numpy()
            rows = {}
            for k, si in enumerate(out.seg_index):
                rows.setdefault(si, []).append(int(toks[k]))
            for si, r in enumerate(grp):
                ver = rows[si]
                st.windows += 1
                cut = next((i for i, (c, v) in enumerate(zip(cand[r], ver)) if c != v), None)
                if cut is None:
                    seqs[r].extend(cand[r])
                    st.committed += len(cand[r])
                else:
                    seqs[r].extend(cand[r][:cut] + [ver[cut]])
                    st.committed += cut + 1
                    st.mismatches += 1
                    st.discarded += len(cand[r]) - cut
