#!/usr/bin/env python3
"""Benchmark of the block-paged KV attention path on one MI355X.

Headline step (timed): one decode tick of the Gemma-style workload -- 32
sequences with context lengths uniform in [512, 4096], 8 query / 2 kv heads,
head_dim 256, bf16, tanh softcap 50: append the tick's 32 new K/V rows into
their cache slots, then run the paged decode over every sequence.  ``value``
is algorithmic HBM bytes per second of the whole step (K/V read once per kv
head, q read, output written, table entries and lengths, the appended rows
read and written).  The pool is replicated R times in HBM and consecutive
steps read different replicas, so that no step is served from the 256 MB
Infinity Cache by its predecessor.  Each step is captured once per replica as
a HIP graph and replayed, as an engine replays its captured decode step.

Also reported on the same line: the decode kernel's roofline (HIP-event
timing of the decode launches inside the timed region), the chunked-prefill
TFLOP/s (the metric's second half), the other decode workloads, and the CPU
oracle timed on the host as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
METRIC = "paged-decode KV GB/s (% HBM peak) + tok/s; paged-prefill TFLOP/s at 1 GPU"
PROFILES = os.path.join(ROOT, "profiles")
# what a kernel's HBM counters depend on: its sources and its argument struct
KERNEL_SOURCES = {
    "decode": (["decode.hip", "slots.hpp", "attn_tile.hpp", "common.hpp"], "DecodeArgs"),
    "prefill": (["prefill.hip", "attn_tile.hpp", "common.hpp"], "PrefillArgs"),
}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--replicas", type=int, default=0, help="pool replicas (0: enough for 1 GiB)")
    p.add_argument("--cpu-seconds", type=float, default=6.0,
                   help="oracle time budget of the headline workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--quick", action="store_true", help="headline step only")
    p.add_argument("--prefill-only", action="store_true",
                   help="only the chunk append and prefill timing (for counter runs)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain device copy of known size (HBM counter calibration)")
    p.add_argument("--timeline-raw", metavar="FILE.npy", default=None,
                   help="with --timeline: also save the raw stamps of the live workgroups")
    p.add_argument("--copy-only", action="store_true",
                   help="only the copy-on-write block copy timing (for counter runs)")
    p.add_argument("--decode-only", metavar="WORKLOAD", default=None,
                   choices=["gemma_decode", "sliding_window_decode", "long_context_splitk"],
                   help="only the decode timing of WORKLOAD (for counter runs)")
    p.add_argument("--partition-size", type=int, default=None,
                   help="with --decode-only: run the split-K decode with this partition size "
                        "(0: the balanced split) instead of the workload's own")
    p.add_argument("--mixed-only", action="store_true",
                   help="time only the mixed batch (one launch, one prefill launch, prefill then "
                        "decode) and print one JSON line")
    p.add_argument("--timeline", metavar="WORKLOAD", default=None,
                   choices=["gemma_decode", "sliding_window_decode",
                            "chunked_prefill_shared_prefix"],
                   help="per-workgroup phase breakdown of one decode launch of WORKLOAD; needs "
                        "the timeline build (PKV_LIBRARY=block_paged_kv_append_amd/libpkv_timeline.so)")
    return p.parse_args()


def source_sha(kind: str) -> str:
    files, args_struct = KERNEL_SOURCES[kind]
    csrc = os.path.join(ROOT, "block_paged_kv_append_amd", "csrc")
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(csrc, "launch.hpp")) as fh:
        m = re.search(r"struct %s \{.*?\n\};" % args_struct, fh.read(), re.S)
    h.update(m.group(0).encode() if m else b"")
    return h.hexdigest()[:16]


def measured_traffic(kind: str, dispatches_per_launch: int = 1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, "hbm_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)[kind]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(kind):
        return None
    return rec["bytes_per_dispatch"] * dispatches_per_launch


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------
def decode_bytes(case) -> int:
    s = 2 if case.dtype == "bf16" else 4
    B, Hq, Hkv, D = case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim
    kv = 0
    blocks = 0
    for L in case.context_lens.tolist():
        n_vis = min(L, case.window) if case.window > 0 else L
        kv += n_vis * Hkv * D * s * 2
        lo = L - n_vis
        blocks += ((L - 1) // 16 - lo // 16 + 1) if L > 0 else 0
    return kv + 2 * B * Hq * D * s + 4 * (B + blocks)


def append_bytes(num_tokens, Hkv, D, s) -> int:
    return 2 * (2 * num_tokens * Hkv * D * s) + 4 * num_tokens


def tick_bytes(case) -> int:
    """A fused decode tick: the decode's bytes, plus the new K and V rows read
    and written into the pool."""
    s = 2 if case.dtype == "bf16" else 4
    return decode_bytes(case) + 2 * (2 * case.num_seqs * case.num_kv_heads * case.head_dim * s)


def prefill_flops(case) -> float:
    pairs = 0
    for b in range(case.num_seqs):
        L, n = int(case.context_lens[b]), int(case.q_lens[b])
        for j in range(n):
            qp = L - n + j
            lo = max(0, qp - case.window + 1) if case.window > 0 else 0
            pairs += qp - lo + 1
    return 4.0 * case.head_dim * case.num_q_heads * pairs


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------
class DecodeBench:
    """Device-resident inputs of one decode workload, replicated R times."""

    def __init__(self, case, replicas, torch, pkv):
        import numpy as np

        self.case, self.torch, self.pkv = case, torch, pkv
        dt = case.dtype
        # enough replicas that 1 GiB is read between two reads of one
        # replica: a call's K/V then comes from HBM, not the 256 MB
        # Infinity Cache (as one layer's cache in an engine, read once per
        # step between the other layers')
        R = replicas or max(2, math.ceil((1 << 30) / decode_bytes(case)))
        self.R = R
        kp = pkv.from_bits(case.k_pool, dt)
        vp = pkv.from_bits(case.v_pool, dt)
        self.kp = torch.cat([kp] * R).contiguous()
        self.vp = torch.cat([vp] * R).contiguous()
        del kp, vp
        NB = case.num_blocks
        bt = case.block_tables.astype(np.int64)
        self.bt = [torch.from_numpy((bt + r * NB).astype(np.int32)).cuda() for r in range(R)]
        self.cl = torch.from_numpy(case.context_lens).cuda()
        self.q = pkv.from_bits(case.q, dt)
        self.out = torch.empty_like(self.q)
        B, Hkv, D = case.num_seqs, case.num_kv_heads, case.head_dim
        # this tick's new token of each sequence sits at position L - 1
        slots = np.array([int(case.block_tables[b, (L - 1) // 16]) * 16 + (L - 1) % 16
                          for b, L in enumerate(case.context_lens.tolist())], dtype=np.int64)
        self.slots = [torch.from_numpy((slots + r * NB * 16).astype(np.int32)).cuda()
                      for r in range(R)]
        g = torch.Generator(device="cuda")
        g.manual_seed(12345)
        tdt = self.q.dtype
        self.k_new = torch.randn(B, Hkv, D, generator=g, device="cuda").to(tdt)
        self.v_new = torch.randn(B, Hkv, D, generator=g, device="cuda").to(tdt)
        ws = pkv.paged_attn_decode_workspace_size(B, Hkv, case.gqa_group, D, case.max_context_len,
                                                  case.partition_size)
        self.ws = torch.zeros(ws, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()

    def decode(self, r):
        c, pkv = self.case, self.pkv
        args = (self.out, self.q, self.kp, self.vp, self.bt[r], self.cl, c.max_context_len, c.scale,
                c.softcap, c.window)
        if c.partition_size:
            pkv.paged_attn_decode_splitk(*args, partition_size=c.partition_size, workspace=self.ws)
        else:
            pkv.paged_attn_decode(*args, workspace=self.ws)

    def append(self, r):
        self.pkv.paged_kv_append(self.k_new, self.v_new, self.slots[r], self.kp, self.vp)

    def tick(self, r):
        """The fused form: append and decode in one launch."""
        c, pkv = self.case, self.pkv
        pkv.paged_attn_decode_append(self.out, self.q, self.k_new, self.v_new, self.kp, self.vp,
                                     self.bt[r], self.cl, c.max_context_len, c.scale, c.softcap,
                                     c.window, partition_size=c.partition_size, workspace=self.ws)

    def two_calls(self, r):
        self.append(r)
        self.decode(r)


def capture(torch, fn):
    """A HIP graph of whatever ``fn`` launches on the current stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def warm(g, torch, seconds=0.4):
    """Replay ``g`` for about ``seconds``: the GPU's clocks ramp up under
    load, and a kernel timed from cold runs several percent slow."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            g.replay()
        torch.cuda.synchronize()


def time_steps(bench, steps, warmup, step, torch):
    """One HIP graph holds R consecutive steps, one per pool replica (as an
    engine's captured decode step holds every layer's attention); each step
    is ``step(r)``: the tick's append and decode.  Returns the wall time of
    ``steps`` steps (``steps / R`` replays, rounded up to whole replays)."""
    def all_steps():
        for r in range(bench.R):
            step(r)

    all_steps()  # eager warm-up
    torch.cuda.synchronize()
    g = capture(torch, all_steps)
    reps = max(1, -(-steps // bench.R))
    warm(g, torch)  # clocks up first, then the W warm-up steps proper
    for _ in range(max(1, -(-warmup // bench.R))):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * steps / (reps * bench.R)


OP_CALLS = 24  # calls per timed graph replay: the replay's own start-up is spread over them


def time_decode_op(bench, iters, torch, op=None, spread=None):
    """Average duration of one decode operation (``op(r)``, by default the
    plain decode): a graph of about OP_CALLS calls cycling over the R pool
    replicas, replayed ``iters`` times, each replay bracketed by HIP events on
    the stream, divided by the calls per replay.  With a dict ``spread``,
    also the 10th and 90th percentiles of those per-replay means."""
    import numpy as np

    op = op or bench.decode
    rounds = max(1, OP_CALLS // bench.R)

    def all_decodes():
        for _ in range(rounds):
            for r in range(bench.R):
                op(r)

    all_decodes()
    torch.cuda.synchronize()
    g = capture(torch, all_decodes)
    warm(g, torch)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record()
        g.replay()
        ev[i][1].record()
    torch.cuda.synchronize()
    per_call = np.array([a.elapsed_time(b) for a, b in ev]) / (rounds * bench.R)
    if spread is not None:  # p10 / p90 of the per-call means of the replays
        spread.update(p10_ms=round(float(np.percentile(per_call, 10)), 5),
                      p90_ms=round(float(np.percentile(per_call, 90)), 5),
                      replays=iters, calls_per_replay=rounds * bench.R)
    return float(np.mean(per_call))


APPEND_REPEAT = 16  # appends per graph replay: one alone is shorter than a launch
PREFILL_REPEAT = 8  # prefills per graph replay (each recomputes the same output)


def time_prefill(case, iters, warmup, torch, pkv, spread=None):
    """Average durations of the chunk append and of the prefill, each replayed
    from its own graph and bracketed by HIP events."""
    import numpy as np

    dt = case.dtype
    kp = pkv.from_bits(case.k_pool, dt)
    vp = pkv.from_bits(case.v_pool, dt)
    k_new, v_new = pkv.from_bits(case.k_new, dt), pkv.from_bits(case.v_new, dt)
    slots = torch.from_numpy(case.slot_mapping).cuda()
    q = pkv.from_bits(case.q, dt)
    out = torch.empty_like(q)
    cu = torch.from_numpy(case.cu_q_lens).cuda()
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(case.context_lens).cuda()

    def append():  # the same rows again: idempotent, and enough work per replay
        for _ in range(APPEND_REPEAT):
            pkv.paged_kv_append(k_new, v_new, slots, kp, vp)

    def prefill():
        for _ in range(PREFILL_REPEAT):
            pkv.paged_attn_prefill(out, q, cu, case.max_q_len, kp, vp, bt, cl,
                                   case.max_context_len, case.scale, case.softcap, case.window)

    append()
    prefill()
    torch.cuda.synchronize()
    ga, gp = capture(torch, append), capture(torch, prefill)
    res = []
    for g in (ga, gp):
        for _ in range(warmup):
            g.replay()
        warm(g, torch)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for i in range(iters):
            ev[i][0].record()
            g.replay()
            ev[i][1].record()
        torch.cuda.synchronize()
        res.append(np.array([a.elapsed_time(b) for a, b in ev]))
    app, pre = res[0] / APPEND_REPEAT, res[1] / PREFILL_REPEAT
    if spread is not None:
        for k, v in (("append", app), ("prefill", pre)):
            spread[k] = {"p10_ms": round(float(np.percentile(v, 10)), 5),
                         "p90_ms": round(float(np.percentile(v, 90)), 5)}
    return float(np.mean(app)), float(np.mean(pre))


COPY_PAIRS = 512  # copy-on-write pairs per call in the block-copy measurement


def time_copy_blocks(bench, iters, torch):
    """Average duration of one paged_kv_copy_blocks call copying COPY_PAIRS
    whole blocks (disjoint random sources and destinations) of the decode
    bench's pools: a graph of one call per pool replica, replayed ``iters``
    times, each replay bracketed by HIP events.  Run after the decode
    timings (it overwrites blocks)."""
    import numpy as np

    case, pkv = bench.case, bench.pkv
    NB = case.num_blocks
    perm = np.random.default_rng(77).permutation(NB)
    n = min(COPY_PAIRS, NB // 2)
    pairs = [(torch.from_numpy((perm[:n] + r * NB).astype(np.int32)).cuda(),
              torch.from_numpy((perm[n:2 * n] + r * NB).astype(np.int32)).cuda())
             for r in range(bench.R)]

    def copies():
        for src, dst in pairs:
            pkv.paged_kv_copy_blocks(src, dst, bench.kp, bench.vp)

    copies()
    torch.cuda.synchronize()
    g = capture(torch, copies)
    warm(g, torch, 0.2)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record()
        g.replay()
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev])) / bench.R
    per_pair = 2 * case.num_kv_heads * case.head_dim * 16 * (2 if case.dtype == "bf16" else 4)
    return ms, n, 2 * n * per_pair  # bytes read + written


def time_mixed(torch, pkv, wl, iters=20):
    """A mixed batch: 4 prefill chunks (2048 cached + 512 new tokens) and 28
    decode rows (contexts uniform in [512, 4096]), 8 q / 2 kv heads, D 256,
    bf16.  Times paged_attn_mixed (one launch: the chunks through the prefill
    body, the decode rows through the balanced decode split beside them) and,
    for comparison, the same batch through one prefill launch, and through a
    prefill launch for the chunks followed by a decode launch for the rows."""
    import numpy as np

    rng = np.random.default_rng(6)
    lens = rng.integers(512, 4097, size=28)
    cached = [2048] * 4 + [int(L) - 1 for L in lens]
    chunk = [512] * 4 + [1] * 28
    c = wl.make_prefill_case(6, cached, chunk, 8, 2, 256, "bf16", scale=1.0 / 16.0, softcap=50.0)
    kp, vp = pkv.from_bits(c.k_pool, "bf16"), pkv.from_bits(c.v_pool, "bf16")
    pkv.paged_kv_append(pkv.from_bits(c.k_new, "bf16"), pkv.from_bits(c.v_new, "bf16"),
                        torch.from_numpy(c.slot_mapping).cuda(), kp, vp)
    q = pkv.from_bits(c.q, "bf16")
    out = torch.empty_like(q)
    cu_all = torch.from_numpy(c.cu_q_lens).cuda()
    cu4 = torch.from_numpy(c.cu_q_lens[:5].copy()).cuda()
    bt = torch.from_numpy(c.block_tables).cuda()
    cl = torch.from_numpy(c.context_lens).cuda()
    ws = torch.zeros(pkv.paged_attn_decode_workspace_size(28, 2, 4, 256, c.max_context_len, 0),
                     dtype=torch.uint8, device="cuda")

    def mixed():
        for _ in range(4):
            pkv.paged_attn_mixed(out, q, cu4, 2048, 512, kp, vp, bt, cl, c.max_context_len,
                                 c.scale, c.softcap, 0, workspace=ws)

    def one_prefill():
        for _ in range(4):
            pkv.paged_attn_prefill(out, q, cu_all, 512, kp, vp, bt, cl, c.max_context_len,
                                   c.scale, c.softcap, 0)

    P = 4 * 512  # the chunks' rows; the decode rows follow them
    bt4, cl4 = bt[4:].contiguous(), cl[4:].contiguous()

    def two_launches():  # the chunks through the prefill, then the rows through the decode
        for _ in range(4):
            pkv.paged_attn_prefill(out[:P], q[:P], cu4, 512, kp, vp, bt[:4], cl[:4],
                                   c.max_context_len, c.scale, c.softcap, 0)
            pkv.paged_attn_decode(out[P:], q[P:], kp, vp, bt4, cl4, c.max_context_len, c.scale,
                                  c.softcap, 0, workspace=ws)

    res = []
    for fn in (mixed, one_prefill, two_launches):
        fn()
        torch.cuda.synchronize()
        g = capture(torch, fn)
        warm(g, torch, 0.2)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        for i in range(iters):
            ev[i][0].record()
            g.replay()
            ev[i][1].record()
        torch.cuda.synchronize()
        res.append(float(np.mean([a.elapsed_time(b) for a, b in ev])) / 4)
    return res[0], res[1], res[2]


def time_eviction(torch, pkv, wl):
    """The decode behind the eviction policies, beside the plain decode of the
    same workload: AttentionSink (4 sink tokens kept beside the 512-token
    window) on the sliding-window workload, and H2O (per-head logits, then the
    per-token attention mass of the step) on the Gemma-style workload."""
    res = {}
    c = wl.sliding_window_decode()
    b = DecodeBench(c, 0, torch, pkv)

    def sink(r):
        pkv.paged_attn_decode_sink_h2o(b.out, b.q, b.kp, b.vp, b.bt[r], b.cl, c.max_context_len,
                                       c.scale, c.softcap, c.window, sink_tokens=4, workspace=b.ws)

    res["attention_sink"] = {"workload": "sliding_window_decode + 4 sink tokens",
                             "ms": round(time_decode_op(b, 20, torch, sink), 5),
                             "plain_decode_ms": round(time_decode_op(b, 20, torch), 5)}
    del b, c
    torch.cuda.empty_cache()
    c = wl.gemma_decode()
    b = DecodeBench(c, 0, torch, pkv)
    S = (c.max_context_len + 15) // 16 * 16  # logit rows: a multiple of 16 >= the longest context
    scores = torch.empty(c.num_seqs, c.num_q_heads, S, device="cuda")
    mass = torch.empty(c.num_seqs, c.num_kv_heads, S, device="cuda")
    lse = torch.empty(c.num_seqs, c.num_q_heads, device="cuda")

    def h2o(r):
        pkv.paged_attn_decode_sink_h2o(b.out, b.q, b.kp, b.vp, b.bt[r], b.cl, c.max_context_len,
                                       c.scale, c.softcap, 0, scores=scores, column_mass=mass,
                                       lse=lse, workspace=b.ws)

    res["h2o_column_mass"] = {"workload": "gemma_decode: logits [32, 8, %d] and mass [32, 2, %d]"
                                          % (S, S),
                              "ms": round(time_decode_op(b, 20, torch, h2o), 5),
                              "plain_decode_ms": round(time_decode_op(b, 20, torch), 5)}
    del b, c, scores, mass
    torch.cuda.empty_cache()
    return res


def copy_rate(torch) -> float:
    """GB/s (bytes read + written) of a plain 1 GiB device copy right now: the
    bandwidth this GPU delivers to a trivial kernel, as context for the rates
    above (it varies from one machine to another)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 20
    del a, b
    torch.cuda.empty_cache()
    return 2 * n / (ms * 1e-3) / 1e9


def _events_ms(torch, fn, reps=10, warm=3):
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def read_rate(torch, pkv):
    """GB/s of a plain sequential read of 2 GiB (the library's read probe),
    the best over 2, 4, 8 and 16 workgroups per compute unit: the highest
    HBM read rate a kernel reaches on this GPU right now.  Returns (best
    GB/s, {workgroups per CU: GB/s})."""
    n = 2 << 30
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    buf = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(3)
    out = torch.empty(16 * cus, dtype=torch.int32, device="cuda")
    rates = {}
    for per_cu in (2, 4, 8, 16):
        ms = _events_ms(torch, lambda: pkv.hbm_read_probe(buf, out, num_wgs=per_cu * cus))
        rates[per_cu] = round(n / (ms * 1e-3) / 1e9, 1)
    del buf, out
    torch.cuda.empty_cache()
    return max(rates.values()), rates


def gather_rate(torch, pkv, bench):
    """GB/s of reading whole blocks of the decode bench's pools (K and V of
    every block of every replica, 32 KiB per block) in a random order (the
    library's gather probe, one and two workgroups per compute unit, the
    better): the decode's access pattern without its arithmetic."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nb = bench.kp.shape[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    order = torch.randperm(nb, generator=g, device="cuda").to(torch.int32)
    out = torch.empty(2 * cus, dtype=torch.int32, device="cuda")
    nbytes = 2 * bench.kp.numel() * bench.kp.element_size()
    best = 0.0
    for per_cu in (1, 2):
        ms = _events_ms(torch, lambda: pkv.hbm_gather_probe(bench.kp, bench.vp, order, out,
                                                          num_wgs=per_cu * cus))
        best = max(best, nbytes / (ms * 1e-3) / 1e9)
    del order, out
    return best


def gemm_rate(torch) -> float:
    """TFLOP/s of a plain 8192^3 bf16 matrix product through torch (hipBLASLt)
    on N(0, 1) operands: the matrix-core rate a tuned library GEMM reaches on
    this GPU right now (the part is power-limited well below its listed
    dense peak on random data), context for the prefill's rate."""
    n = 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    a = torch.randn(n, n, generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, generator=g, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        c = a @ b
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del a, b, c
    torch.cuda.empty_cache()
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def mfma_rate(torch, pkv):
    """The matrix-core rate this GPU sustains with every SIMD issuing
    back-to-back bf16 32x32x16 products (the library's probe, one workgroup of
    four waves per compute unit, about 2 ms), and the shader clock the SIMDs
    ran at: (TFLOP/s, MHz, cycles per product), all medians over workgroups
    except the rate (all products over the launch's HIP-event time)."""
    import numpy as np

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 2000
    stamps = torch.zeros(4 * cus, dtype=torch.int64, device="cuda")
    pkv.mfma_rate_probe(stamps, iters, num_wgs=cus)  # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    pkv.mfma_rate_probe(stamps, iters, num_wgs=cus)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    s = stamps.cpu().numpy().reshape(cus, 4).astype(np.float64)
    cycles, ticks = s[:, 1] - s[:, 0], s[:, 3] - s[:, 2]
    flops = cus * 4 * iters * 8 * 32768.0
    return (flops / (ms * 1e-3) / 1e12, float(np.median(cycles / ticks * 100.0)),
            float(np.median(cycles / (iters * 8))))


def calibrate_copy(torch):
    """A plain device-to-device copy of 1 GiB, 10 times: the reference for
    scaling the HBM FETCH_SIZE / WRITE_SIZE counters."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 10}))


def prefill_timeline(name, torch, pkv, wl, replays=40, raw_out=None):
    """Per-workgroup entry and exit stamps of one prefill launch of the named
    workload, taken by the timeline build of the library: the shader-clock
    counter (s_memtime) and the constant-rate counter (s_memrealtime) at entry
    and after the pair merge, so the line gives each workgroup's duration, the
    clock it ran at, and its matrix-core cycles at the nominal 32 cycles per
    32x32x16 product against its cycles."""
    import ctypes

    import numpy as np

    lib = pkv.load_library()
    if not hasattr(lib, "pkv_timeline_set"):
        raise SystemExit("--timeline needs the timeline build: "
                         "PKV_LIBRARY=block_paged_kv_append_amd/libpkv_timeline.so")
    lib.pkv_timeline_set.argtypes = [ctypes.c_void_p]
    lib.pkv_timeline_set.restype = None
    lib.pkv_timeline_clock_khz.restype = ctypes.c_int
    khz = lib.pkv_timeline_clock_khz()
    case = getattr(wl, name)()
    dt = case.dtype
    kp, vp = pkv.from_bits(case.k_pool, dt), pkv.from_bits(case.v_pool, dt)
    q = pkv.from_bits(case.q, dt)
    out = torch.empty_like(q)
    cu = torch.from_numpy(case.cu_q_lens).cuda()
    bt = torch.from_numpy(case.block_tables).cuda()
    cl = torch.from_numpy(case.context_lens).cuda()
    buf = torch.zeros(TL_WGS * TL_STAMPS, dtype=torch.int64, device="cuda")
    lib.pkv_timeline_set(buf.data_ptr())

    def calls():
        for _ in range(PREFILL_REPEAT):
            pkv.paged_attn_prefill(out, q, cu, case.max_q_len, kp, vp, bt, cl,
                                   case.max_context_len, case.scale, case.softcap, case.window)

    calls()
    torch.cuda.synchronize()
    g = capture(torch, calls)
    warm(g, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    buf.zero_()
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    per_call_us = e0.elapsed_time(e1) * 1e3 / (replays * PREFILL_REPEAT)
    lib.pkv_timeline_set(None)
    st = buf.view(TL_WGS, TL_STAMPS).cpu().numpy().astype(np.int64)
    live = st[:, 3] != 0
    s = st[live]
    if raw_out:
        np.save(raw_out, s[:, :8])
    cycles = (s[:, 1] - s[:, 0]).astype(np.float64)
    wg_us = (s[:, 3] - s[:, 2]) * 1e3 / khz
    mhz = cycles / wg_us
    stages = s[:, 4].astype(np.float64)
    products = stages * (case.head_dim // 8)  # per SIMD: D/16 + D/16 per stage
    span_us = float((s[:, 3].max() - s[:, 2].min()) * 1e3 / khz)

    def pct(x):
        x = np.asarray(x, dtype=np.float64)
        return {k: round(float(np.percentile(x, q_)), 3)
                for k, q_ in (("min", 0), ("p10", 10), ("p50", 50), ("p90", 90), ("max", 100))}

    tiles = s[:, 5]
    by_tile = {int(t): round(float(wg_us[tiles == t].mean()), 2) for t in np.unique(tiles)}
    return {
        "timeline": name, "workgroups": int(live.sum()), "clock_khz": khz,
        "per_call_us_events": round(per_call_us, 2), "span_us": round(span_us, 2),
        "shader_clock_mhz": pct(mhz), "workgroup_us": pct(wg_us),
        "workgroup_cycles": pct(cycles), "stages": pct(stages),
        "matrix_core_frac_nominal": pct(products * 32 / cycles),
        "workgroup_us_by_tile": by_tile,
    }


# ---------------------------------------------------------------------------
# timeline: where one decode launch spends its time (timeline build only)
# ---------------------------------------------------------------------------
TL_WGS, TL_STAMPS = 4096, 32  # the library's timeline buffer geometry


def timeline(name, torch, pkv, wl, replays=40, raw_out=None):
    """Phase stamps of every workgroup of one decode launch of the named
    workload, taken by the timeline build of the library (s_memrealtime, one
    lane per workgroup; the block-loop end per wave).  The launch is the last
    of a graph of calls over the pool replicas, replayed like the bench's
    timed steps (the Gemma-style workload runs its fused tick)."""
    import ctypes

    import numpy as np

    lib = pkv.load_library()
    if not hasattr(lib, "pkv_timeline_set"):
        raise SystemExit("--timeline needs the timeline build: "
                         "PKV_LIBRARY=block_paged_kv_append_amd/libpkv_timeline.so")
    lib.pkv_timeline_set.argtypes = [ctypes.c_void_p]
    lib.pkv_timeline_set.restype = None
    lib.pkv_timeline_clock_khz.restype = ctypes.c_int
    khz = lib.pkv_timeline_clock_khz()
    case = getattr(wl, name)()
    b = DecodeBench(case, 0, torch, pkv)
    op = b.tick if name == "gemma_decode" else b.decode
    buf = torch.zeros(TL_WGS * TL_STAMPS, dtype=torch.int64, device="cuda")
    lib.pkv_timeline_set(buf.data_ptr())

    def calls():
        for r in range(b.R):
            op(r)

    calls()
    torch.cuda.synchronize()
    g = capture(torch, calls)
    warm(g, torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    buf.zero_()
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    per_call_us = e0.elapsed_time(e1) * 1e3 / (replays * b.R)
    lib.pkv_timeline_set(None)
    st = buf.view(TL_WGS, TL_STAMPS).cpu().numpy().astype(np.int64)
    live = (st[:, 11] != 0) & (st[:, 2] != 0)  # workgroups that ran a piece
    s = st[live]
    t0 = s[:, 0].min()
    us = lambda col: (s[:, col] - t0) * 1e3 / khz  # noqa: E731
    loop_end = (s[:, 4:8].max(axis=1) - t0) * 1e3 / khz
    loop_first = (s[:, 4:8].min(axis=1) - t0) * 1e3 / khz
    # count-in and merge of the last piece (stamps of an earlier piece are older than its combine)
    merged = s[:, 10] > s[:, 8]

    def pct(x):
        x = np.asarray(x, dtype=np.float64)
        if x.size == 0:
            return None
        return {k: round(float(np.percentile(x, q)), 2)
                for k, q in (("min", 0), ("p10", 10), ("p50", 50), ("p90", 90), ("max", 100))}

    split = s[:, 9] > s[:, 8]  # the last piece was split: it counted in
    xcd = np.nonzero(live)[0] % 8
    res = {
        "timeline": name, "workgroups": int(live.sum()), "clock_khz": khz,
        "per_call_us_events": round(per_call_us, 2),
        "span_us": round(float(us(11).max()), 2),
        "phases_us_from_first_entry": {
            "entry": pct(us(0)), "setup_done": pct(us(1)), "first_copies_issued": pct(us(2)),
            "first_block_landed": pct(us(3)), "block_loop_done_last_wave": pct(loop_end),
            "waves_combined": pct(us(8)), "count_in_done": pct(us(9)[split]),
            "merge_done": pct(us(10)[merged]), "exit": pct(us(11))},
        "durations_us": {
            "setup": pct(us(1) - us(0)), "setup_to_first_copy": pct(us(2) - us(1)),
            "first_copy_latency": pct(us(3) - us(2)),
            "wave_spread_at_loop_end": pct(loop_end - loop_first),
            "combine_after_last_wave": pct(us(8) - loop_end),
            "count_in": pct((us(9) - us(8))[split]),
            "merge": pct((us(10) - us(9))[merged]),
            "first_piece_entry_to_issue_loop": pct(us(13) - us(12)),
            "first_piece_issue_loop": pct(us(2) - us(13)),
            "first_piece_table_and_q_wait": pct(us(16) - us(13)),
            "first_piece_copy_issue": pct(us(2) - us(16)),
            "combine_barrier_after_last_wave": pct(us(17) - loop_end),
            "combine_lds_write": pct(us(18) - us(17)),
            "combine_fold_and_store": pct(us(8) - us(18)),
            "count_in_store_wait": pct((us(19) - us(8))[split]),
            "count_in_atomic": pct((us(9) - us(19))[split]),
            "second_piece_entry_to_copies_issued": pct((us(15) - us(14))[s[:, 14] != 0])},
        "merging_workgroups": int(merged.sum()),
        "two_piece_workgroups": int((s[:, 14] != 0).sum()),
        "entry_by_xcd_us": {int(x): pct(us(0)[xcd == x]) for x in range(8)},
    }
    if raw_out:
        np.save(raw_out, st[live])
    del b
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores
# ---------------------------------------------------------------------------
def _host_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def cpu_baseline(case, budget_s, runs=None):
    """The float64 oracle's decode of the whole workload on the host cores:
    passes until ``budget_s`` seconds (or exactly ``runs`` passes, the median
    reported), as algorithmic GB/s."""
    import numpy as np

    import oracle

    threads = _host_threads()
    per_pass = decode_bytes(case)
    times, t0 = [], time.perf_counter()
    while True:
        t = time.perf_counter()
        oracle.decode(case.q, case.k_pool, case.v_pool, case.block_tables, case.context_lens,
                      case.scale, case.softcap, case.window, case.dtype)
        times.append(time.perf_counter() - t)
        el = time.perf_counter() - t0
        if (runs and len(times) >= runs) or (not runs and (el >= budget_s or len(times) >= 1000)):
            break
    if runs:
        sec = float(np.median(times))
        how = f"median of {len(times)} passes over the full workload (all {case.num_seqs} " \
              f"sequences), {sec:.2f} s each"
    else:
        sec = el / len(times)
        how = f"full workload (all {case.num_seqs} sequences), {len(times)} passes in {el:.1f} s"
    return {"value": round(per_pass / sec / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{how}; float64 numpy, BLAS threads {threads}, "
                      f"host affinity {len(os.sched_getaffinity(0))} cpus"}


def cpu_baseline_prefill(case):
    """The float64 oracle's prefill of the whole chunked-prefill workload (the
    chunk already appended), one pass, as algorithmic GFLOP/s."""
    import oracle

    threads = _host_threads()
    kr, vr = oracle.append(case.k_new, case.v_new, case.slot_mapping, case.k_pool, case.v_pool,
                           case.dtype)
    t = time.perf_counter()
    oracle.prefill(case.q, case.cu_q_lens, kr, vr, case.block_tables, case.context_lens,
                   case.scale, case.softcap, case.window, case.dtype)
    sec = time.perf_counter() - t
    return {"value": round(prefill_flops(case) / sec / 1e9, 3), "unit": "GFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"one pass over the full workload (all {case.num_seqs} chunks), {sec:.2f} s; "
                      f"float64 numpy, BLAS threads {threads}, host affinity "
                      f"{len(os.sched_getaffinity(0))} cpus"}


# ---------------------------------------------------------------------------
def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: the path runs on one GPU; --gpus {args.gpus} is not supported "
              f"(use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import block_paged_kv_append_amd as pkv
    from block_paged_kv_append_amd import workloads as wl

    pkv.load_library()  # raises if libpkv.so is missing: there is no fallback
    if args.timeline:
        fn = prefill_timeline if args.timeline == "chunked_prefill_shared_prefix" else timeline
        print(json.dumps(fn(args.timeline, torch, pkv, wl, raw_out=args.timeline_raw)), flush=True)
        return
    if args.copy_only:
        c = wl.gemma_decode()
        b = DecodeBench(c, 0, torch, pkv)
        ms, pairs, nbytes = time_copy_blocks(b, 20, torch)
        print(json.dumps({"copy_blocks_pairs": pairs, "ms": round(ms, 5),
                          "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes}))
        return
    if args.decode_only:
        c = getattr(wl, args.decode_only)()
        if args.partition_size is not None:
            c.partition_size = args.partition_size
        b = DecodeBench(c, 0, torch, pkv)
        ms = time_decode_op(b, 20, torch)
        print(json.dumps({"decode_only": c.name, "partition_size": c.partition_size,
                          "ms": round(ms, 5),
                          "gbs": round(decode_bytes(c) / (ms * 1e-3) / 1e9, 1),
                          "algorithmic_bytes": decode_bytes(c), "pool_replicas": b.R}))
        return
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.mixed_only:
        mx_ms, one_ms, two_ms = time_mixed(torch, pkv, wl)
        print(json.dumps({"mixed_call_ms": round(mx_ms, 5), "one_prefill_launch_ms": round(one_ms, 5),
                          "prefill_then_decode_ms": round(two_ms, 5)}))
        return
    if args.prefill_only:
        pc = wl.chunked_prefill_shared_prefix()
        app_ms, pre_ms = time_prefill(pc, 20, 3, torch, pkv)
        print(json.dumps({"prefill_ms": round(pre_ms, 5), "append_ms": round(app_ms, 5)}))
        return

    t_setup = time.perf_counter()
    case = wl.gemma_decode()
    bench = DecodeBench(case, args.replicas, torch, pkv)
    print(f"# setup {time.perf_counter() - t_setup:.1f}s, pool replicas {bench.R}", file=sys.stderr,
          flush=True)

    wall = time_steps(bench, args.steps, args.warmup, bench.tick, torch)
    ms_per_step = wall * 1e3 / args.steps
    tbytes = tick_bytes(case)
    value = tbytes / (ms_per_step * 1e-3) / 1e9
    kspread = {}
    kern_avg_ms = time_decode_op(bench, max(10, args.steps // bench.R), torch, bench.tick, kspread)
    achieved = tbytes / (kern_avg_ms * 1e-3) / 1e9
    traffic = measured_traffic("decode")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gemma_decode: 32 seqs, ctx U[512,4096], 8q/2kv heads, D256, bf16, "
                               "softcap 50, block 16; step = one decode tick: the 32 new "
                               "tokens appended and decoded in one launch",
                   "num_seqs": case.num_seqs, "context_tokens": int(case.context_lens.sum()),
                   "pool_replicas": bench.R},
        "tok_per_s": round(case.num_seqs / (ms_per_step * 1e-3), 1),
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "paged_attn_decode_append: decode_kernel (balanced split, "
                               "fused append, in-launch merge)",
                     "kernel_ms": round(kern_avg_ms, 5), "kernel_spread": kspread,
                     "algorithmic_bytes": tbytes},
    }

    if not args.quick:
        # the same tick as two launches (append, then decode), and the decode alone
        two_ms = time_steps(bench, args.steps, args.warmup, bench.two_calls, torch) * 1e3 / args.steps
        dec_ms = time_decode_op(bench, max(10, args.steps // bench.R), torch)
        line["step_forms"] = {"fused_ms": round(ms_per_step, 5),
                              "append_then_decode_ms": round(two_ms, 5),
                              "decode_only_ms": round(dec_ms, 5),
                              "decode_only_gbs": round(decode_bytes(case) / (dec_ms * 1e-3) / 1e9, 1)}
        extra = {}
        pc = wl.chunked_prefill_shared_prefix()
        pspread = {}
        app_ms, pre_ms = time_prefill(pc, 40, 3, torch, pkv, pspread)
        flops = prefill_flops(pc)
        tf = flops / (pre_ms * 1e-3) / 1e12
        ab = append_bytes(pc.num_q_tokens, pc.num_kv_heads, pc.head_dim, 2)
        line["prefill"] = {
            "workload": "chunked_prefill_shared_prefix: 8 seqs x (2048 cached, first 1024 shared) "
                        "+ 512-token chunk, 8q/2kv heads, D256, bf16, causal",
            "tflops": round(tf, 2), "ms": round(pre_ms, 5), "spread": pspread["prefill"],
            "flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill")},
            "append": {"ms": round(app_ms, 5), "gbs": round(ab / (app_ms * 1e-3) / 1e9, 1),
                       "hbm_frac": round(ab / (app_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "spread": pspread["append"], "bytes": ab},
        }
        if not args.no_cpu_baseline:
            line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(pc)
        del pc
        cb_ms, cb_pairs, cb_bytes = time_copy_blocks(bench, 20, torch)
        line["copy_blocks"] = {"pairs": cb_pairs, "ms": round(cb_ms, 5),
                               "gbs": round(cb_bytes / (cb_ms * 1e-3) / 1e9, 1), "bytes": cb_bytes,
                               "pool": "gemma_decode (2 kv heads, D256, bf16: 32 KiB per pair)"}
        mx_ms, one_ms, two_ms = time_mixed(torch, pkv, wl)
        line["mixed_batch"] = {
            "workload": "4 prefill chunks (2048 cached + 512) + 28 decode rows (ctx U[512,4096]), "
                        "8q/2kv heads, D256, bf16, softcap 50",
            "mixed_call_ms": round(mx_ms, 5), "one_prefill_launch_ms": round(one_ms, 5),
            "prefill_then_decode_ms": round(two_ms, 5)}
        for maker in (wl.sliding_window_decode, wl.long_context_splitk):
            c = maker()
            b = DecodeBench(c, 0, torch, pkv)
            sp = {}
            ms = time_decode_op(b, 40, torch, spread=sp)
            gbs = decode_bytes(c) / (ms * 1e-3) / 1e9
            extra[c.name] = {"ms": round(ms, 5), "spread": sp, "gbs": round(gbs, 1),
                             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                             "tok_per_s": round(c.num_seqs / (ms * 1e-3), 1),
                             "algorithmic_bytes": decode_bytes(c), "pool_replicas": b.R,
                             "entry": "splitk P=%d" % c.partition_size if c.partition_size else "balanced"}
            if not args.no_cpu_baseline:
                extra[c.name]["cpu_baseline"] = cpu_baseline(c, 0, runs=1 if c.partition_size else 3)
            del b, c
            torch.cuda.empty_cache()
        line["other_workloads"] = extra
        line["eviction_policies"] = time_eviction(torch, pkv, wl)

    if not args.quick:
        line["box_copy_gbs"] = round(copy_rate(torch), 1)
        rr, rr_all = read_rate(torch, pkv)
        line["box_read_gbs"] = round(rr, 1)
        line["box_read_gbs_by_wgs_per_cu"] = rr_all
        line["roofline"]["frac_of_box_read"] = round(achieved / rr, 4)
        gbr = gather_rate(torch, pkv, bench)
        line["box_block_gather_gbs"] = round(gbr, 1)
        line["roofline"]["frac_of_box_block_gather"] = round(achieved / gbr, 4)
        gr = gemm_rate(torch)
        line["box_gemm_tflops"] = round(gr, 1)
        line["prefill"]["roofline"]["frac_of_box_gemm"] = round(line["prefill"]["tflops"] / gr, 4)
        mr, mhz, cpp = mfma_rate(torch, pkv)
        line["box_mfma_tflops"] = round(mr, 1)
        line["box_mfma_clock_mhz"] = round(mhz)
        line["box_mfma_cycles_per_product"] = round(cpp, 2)
        line["prefill"]["roofline"]["frac_of_box_mfma"] = round(line["prefill"]["tflops"] / mr, 4)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
