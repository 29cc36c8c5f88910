"""Benchmark of the int2 draft LM head on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-bands]
    python bench.py --traffic-probe    # short run for rocprofv3 counter passes (see below)

A step is one call of the head's per-call entry point i2h_head over one batch: the coarse int2
pass with its fused block top-8 emit (which sums the groups of x itself), then the top-32
selection, exact bf16 rerank and argmax in one kernel, enqueued on one stream with no host
synchronisation. The same kernels enqueued through their own entry points (two calls per step)
are timed beside it (`us_per_call_separate_entries`). The coarse kernel is also timed alone,
back to back, for the roofline. The workload is one rank's
vocab slice, x[1, 5120] @ W[5120, 124160] (the draft-slot shape), with inputs resident in HBM.
The stored head (packed codes + scales, 178.8 MB) fits in the 256 MB last-level cache, so the
steps rotate over COPIES independent copies of it (2.1 GB) and every step reads its copy from
HBM. The quantise+pack of the bf16 weight is a load-time step and is timed on its own.
Before the first timed region the head runs PREWARM_S seconds of untimed calls: the GPU sits idle
while the weight is generated on the host, and the first tens of milliseconds of calls after that
run several µs slower per call than the rest.

Prints one JSON line. `value` is the head's algorithmic HBM bytes per call divided by the
measured time per call (GB/s); `us_per_call` is the same time, `us_per_call_p10_p50_p90` its
spread over single calls (HIP events between calls). `us_per_call_graph` is the same call
(i2h_head) replayed from a HIP graph holding one call per cold copy. `device` names the GPU, the
HIP version and the compute-unit count; `roofline.copy_gbps_measured` is torch's device copy over
512 MiB on the same box (read + write), the practical HBM rate beside the 8 TB/s peak. `roofline` covers the coarse
kernel, the dominant one, timed with HIP events on the launch stream over the timed region.
`cpu_baseline` times the oracle (test infrastructure, CPU) on the same workload.
`dropin_logits` times the drop-in logits row at the same M: coarse pass with its bf16 row, the
fused tail with its selection and exact scores, and i2h_logits writing the exact scores back
(argmax caller, in place) or over a -inf row (top-k caller), per call and the write-back alone.
`fp8_source` times the same weights as an FP8 e4m3 per-row-scale head: its load-time pack, and the
fused tail reranking against the FP8 rows beside the bf16 one (back-to-back launches).
`int4_head` times the int4 head on the same weights at KCAND = 1 (pack; xsum + int4 coarse +
fused tail per call; the int4 coarse kernel alone, 6-copy rotation) and, with the CPU baseline,
how often its argmax equals the dense bf16 argmax on the match rows (beside the int2 head's).
`ablations.selection` sets the block candidates against a token-level top-R over the whole bf16
coarse row (i2h_select_tokens, then the exact rerank and argmax): per call, the tail alone and the
selection alone, with the token-level path's argmax agreement with the dense bf16 argmax.
`ablations.coarse_variants` times one coarse kernel family in four forms that differ in one
property each (the design: group 128, quarter-split, scale on the accumulator; group 64;
contiguous-4 bytes; dequantised weight tile) at M = 1 and 16 on cold copies, with each pack.
`bands` times the per-call path and the coarse kernel alone at M = 16, 32, 64 on the same slice;
`full_vocab_top16` the unsharded 248320-row vocabulary with the top-16 caller: the GPU pack of its
bf16 weight, and one i2h_head call at each M in (1, 2, 4, 8, 16, 32, 64, 72) on cold copies.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/call + HBM GB/s, int2 head 5120×124160 at M=1/16/64; argmax match %"
WORKLOAD = "draft_slot_m1_k5120_n124160"
COPIES = 12
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFS = 2500.0
KC, R = 8, 32
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "coarse_traffic.json")
COARSE_SRC = os.path.join(ROOT, "bit_quantized_lm_int2_amd", "csrc", "coarse.hip")


def head_bytes(M, N, K, kc=KC, R_=R, k=1, own_sums=False):
    """Algorithmic HBM bytes of one call, per kernel: every input the step must read and every
    output it must write once (packed codes, S, ZS, x, the group sums, the block candidates
    written by the coarse kernel and read by the selection, the selection, the gathered bf16
    weight rows, the results). With own_sums the coarse kernel sums the groups of x itself and
    there is no group-sum array."""
    KG = K // 128
    nblk = (N + 63) // 64
    cand = M * nblk * kc * 8
    stored = N * K // 4 + 2 * N * KG * 2
    b = {
        "xsum": 0 if own_sums else M * K * 2 + M * KG * 4,
        "coarse": stored + M * K * 2 + (0 if own_sums else M * KG * 4) + cand,
        "select": cand + M * R_ * 4,
        "rerank_topk": M * R_ * 4 + M * R_ * K * 2 + M * K * 2 + M * k * 8,
    }
    b["total"] = sum(b.values())
    return b


COARSE_SOURCES = ("coarse.hip", "coarse_tile.hip", "dequant.h", "device_util.h")


def coarse_source_hash():
    h = hashlib.sha256()
    for name in COARSE_SOURCES:
        with open(os.path.join(ROOT, "bit_quantized_lm_int2_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(M):
    """HBM bytes (read + write) per coarse call from the committed rocprofv3 counter runs, if they
    were taken on the current coarse kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != coarse_source_hash():
        return None
    return t.get("per_call_bytes", {}).get(str(M))


class Head:
    """Preallocated buffers and prebuilt ctypes arguments for one M, so a step enqueues five
    launches with no allocation and little host work."""

    def __init__(self, i2h, torch, x, copies, W, M, N, K):
        self.lib = i2h.lib()
        self.x = x
        self.own_sums = i2h.coarse_sums_x(M, K)
        dev = x.device
        KG = K // 128
        nblk = (N + 63) // 64
        self.xs = torch.empty(M, KG, dtype=torch.float32, device=dev)
        self.cs = torch.empty(M, nblk * KC, dtype=torch.float32, device=dev)
        self.ci = torch.empty(M, nblk * KC, dtype=torch.int32, device=dev)
        self.sel = torch.empty(M, R, dtype=torch.int32, device=dev)
        self.ex = torch.empty(M, R, dtype=torch.float32, device=dev)
        self.oi = torch.empty(M, 1, dtype=torch.int32, device=dev)
        self.ov = torch.empty(M, 1, dtype=torch.float32, device=dev)
        ws_n = i2h.workspace_bytes(M, N, K, KC, R)
        self.ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
        s = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        self.stream = s
        self.a_xsum = (P(x), M, K, P(self.xs), s)
        xs_arg = None if self.own_sums else P(self.xs)
        self.a_coarse = [(P(x), xs_arg, M, P(p), P(S), P(Z), N, K, KC, P(self.cs), P(self.ci), None, s)
                         for (p, S, Z) in copies]
        self.a_select = (P(self.cs), P(self.ci), M, nblk, KC, R, P(self.sel), s)
        self.a_rerank = (P(x), M, P(W), W.stride(0), N, K, P(self.sel), R, 1, P(self.ex), P(self.oi),
                         P(self.ov), s)
        self.a_srr = (P(self.cs), P(self.ci), M, nblk, KC, R, P(x), P(W), W.stride(0), N, K, 1, None, None,
                      P(self.oi), P(self.ov), s)
        self.a_head = [(P(x), M, P(p), P(S), P(Z), P(W), W.stride(0), N, K, KC, R, 1, P(self.oi), P(self.ov),
                        None, P(self.ws), ws_n, s) for (p, S, Z) in copies]
        # the drop-in logits row: coarse with its bf16 row, the tail with its selection and exact
        # scores, then the write-back in place (argmax caller) or over -inf (top-k caller)
        self.y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        self.a_coarse_y = [(P(x), xs_arg, M, P(p), P(S), P(Z), N, K, KC, P(self.cs), P(self.ci), P(self.y), s)
                           for (p, S, Z) in copies]
        self.a_srr_sel = (P(self.cs), P(self.ci), M, nblk, KC, R, P(x), P(W), W.stride(0), N, K, 1, P(self.sel),
                          P(self.ex), P(self.oi), P(self.ov), s)
        # token-level selection over the coarse row (the alternative to block candidates)
        nws = i2h.lib().i2h_select_tokens_workspace_bytes(M, N, R)
        self.ws_tok = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        self.a_seltok = (P(self.y), M, N, R, P(self.sel), P(self.ws_tok) if nws > 0 else None, nws, s)
        self.a_rr_sel = (P(x), M, P(W), W.stride(0), N, K, P(self.sel), R, 1, None, P(self.oi), P(self.ov), s)
        self.a_logits = {topk: (None if topk else P(self.y), M, N, P(self.sel), P(self.ex), R, int(topk), None, 0,
                                P(self.y), 1, s) for topk in (False, True)}

    def step(self, i, ev0=None, ev1=None):
        L = self.lib
        st = 0 if self.own_sums else L.i2h_xsum(*self.a_xsum)
        if ev0 is not None:
            ev0.record()
        st |= L.i2h_coarse_topk(*self.a_coarse[i % len(self.a_coarse)])
        if ev1 is not None:
            ev1.record()
        st |= L.i2h_select_rerank_topk(*self.a_srr)
        if st:
            raise RuntimeError(f"libi2h status {st}")

    def coarse_only(self, torch, n, first=0):
        """Mean time of n back-to-back coarse launches (rotating cold copies), by HIP events on the
        launch stream: the per-launch duration the roofline uses."""
        L = self.lib
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            if L.i2h_coarse_topk(*self.a_coarse[(first + i) % len(self.a_coarse)]):
                raise RuntimeError("libi2h coarse launch failed")
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    def dropin(self, i, topk=False):
        L = self.lib
        st = 0 if self.own_sums else L.i2h_xsum(*self.a_xsum)
        coarse = self.a_coarse if topk else self.a_coarse_y  # a top-k caller needs no coarse row
        st |= L.i2h_coarse_topk(*coarse[i % len(coarse)])
        st |= L.i2h_select_rerank_topk(*self.a_srr_sel)
        st |= L.i2h_logits(*self.a_logits[topk])
        if st:
            raise RuntimeError(f"libi2h status {st}")

    def token_level(self, i):
        """One call with token-level selection: coarse with its bf16 row, the top-R of the row,
        then the exact rerank and argmax of those R tokens."""
        L = self.lib
        st = 0 if self.own_sums else L.i2h_xsum(*self.a_xsum)
        st |= L.i2h_coarse_topk(*self.a_coarse_y[i % len(self.a_coarse_y)])
        st |= L.i2h_select_tokens(*self.a_seltok)
        st |= L.i2h_rerank_topk(*self.a_rr_sel)
        if st:
            raise RuntimeError(f"libi2h status {st}")

    def logits_only(self, torch, n, topk=False):
        """Mean time of n back-to-back i2h_logits calls (row pass + write-back) by HIP events."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            if self.lib.i2h_logits(*self.a_logits[topk]):
                raise RuntimeError("libi2h logits launch failed")
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    def fused(self, i):
        st = self.lib.i2h_head(*self.a_head[i % len(self.a_head)])
        if st:
            raise RuntimeError(f"libi2h status {st}")


def back_to_back_us(torch, fn, steps, warmup):
    """Mean µs of `steps` back-to-back calls of fn() (each enqueues launches and returns a
    libi2h status), by HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        if fn():
            raise RuntimeError("libi2h launch failed")
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / steps


PREWARM_S = 0.3


def prewarm(torch, fn, seconds=PREWARM_S):
    """Untimed calls fn(i) for about `seconds` of wall time (synchronised every 100 calls)."""
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(100):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def time_steps(torch, fn, steps, warmup, events=False):
    """(seconds per step by host clock around a synchronised loop, mean coarse ms by events)."""
    for i in range(warmup):
        fn(i, None, None) if events else fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)] if events else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if events:
            fn(warmup + i, *evs[i])
        else:
            fn(warmup + i)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    coarse_ms = None
    if events:
        coarse_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    return dt, coarse_ms


def call_percentiles(torch, np, fn, n, first):
    """(p10, p50, p90) µs of n consecutive calls of fn(i) (each enqueues one call), from a chain of
    HIP events between calls on the current stream (each interval holds one whole call)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(n):
        fn(first + i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    d = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n)])
    return [round(float(v), 2) for v in np.percentile(d, [10, 50, 90])]


def copy_gbps(torch, dev, nbytes=512 << 20, reps=10):
    """Device-to-device copy bandwidth (bytes read + written per second, GB/s) of torch's copy
    kernel over a 512 MiB buffer: the box's practical HBM rate, for context beside the 8 TB/s
    peak."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    del src, dst
    return round(2 * nbytes / us / 1e3, 1)


def device_info(torch):
    """GPU name and HIP runtime version."""
    return {"name": torch.cuda.get_device_name(0), "hip": torch.version.hip,
            "compute_units": torch.cuda.get_device_properties(0).multi_processor_count}


def to_dev_bits(torch, np, b, dev):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)


def traffic_probe(torch, i2h, si, dev):
    """Launches for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes: the coarse kernel on the timed
    workload at M = 1, 16, 32, 64 (cold weight copies, 6 launches each), and a plain device copy of a
    512 MiB buffer (4 launches) whose counter readings give the bytes-per-count factor."""
    cfg = si.WORKLOADS[WORKLOAD]
    K, N = cfg["K"], cfg["N"]
    W = si.gen_weight(N, K).to(dev)
    packed, S, ZS = i2h.pack(W)
    del W
    copies = [(packed, S, ZS)] + [(packed.clone(), S.clone(), ZS.clone()) for _ in range(COPIES - 1)]
    x_all = si.gen_x(64, K, outliers=cfg["outliers"]).to(dev)
    for M in (1, 16, 32, 64):
        x = x_all[:M].contiguous()
        xs = None if i2h.coarse_sums_x(M, K) else i2h.xsum(x)
        for i in range(6):
            p, a, b = copies[(i * 5 + M) % COPIES]
            i2h.coarse_topk(x, xs, p, a, b, kcand=KC)
        torch.cuda.synchronize()
    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_probe": True, "copy_bytes": src.numel(), "M": [1, 16, 32, 64]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bands", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only launch the coarse kernel 6 times per M in (1, 16, 32, 64) on cold weight copies, "
                         "then copy a 512 MiB buffer 4 times (the calibration kernel for HBM byte counters)")
    ap.add_argument("--match-rows", type=int, default=32)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_lm_int2_amd as i2h
    import synth_inputs as si

    i2h.lib()
    dev = torch.device("cuda:0")
    if args.traffic_probe:
        traffic_probe(torch, i2h, si, dev)
        return
    cfg = si.WORKLOADS[WORKLOAD]
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731

    log(f"[bench] generating W [{N}, {K}] and x")
    Wc = si.gen_weight(N, K)
    W = Wc.to(dev)
    nrows = max(args.match_rows, 64)
    x_all_c = si.gen_x(nrows, K, outliers=cfg["outliers"])
    x_all = x_all_c.to(dev)

    # load-time pack, timed on its own
    packed, S, ZS = i2h.pack(W)
    torch.cuda.synchronize()
    pk = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        i2h.pack(W, out=(packed, S, ZS))
        b.record()
        torch.cuda.synchronize()
        pk.append(a.elapsed_time(b) * 1e3)
    pack_us = float(np.median(pk))
    pack_bytes = N * K * 2 + N * K // 4 + 2 * N * (K // 128) * 2
    copies = [(packed, S, ZS)] + [(packed.clone(), S.clone(), ZS.clone()) for _ in range(COPIES - 1)]
    torch.cuda.synchronize()

    def measure(Mb, steps, warmup, warm_s=0.0):
        x = x_all[:Mb].contiguous()
        h = Head(i2h, torch, x, copies, W, Mb, N, K)
        if warm_s > 0:
            prewarm(torch, h.fused, warm_s)
        dt, _ = time_steps(torch, h.step, steps, warmup)
        dt_fused, _ = time_steps(torch, h.fused, steps, warmup)
        h.coarse_only(torch, warmup)
        coarse_ms = h.coarse_only(torch, steps, warmup) * 1e-3
        torch.cuda.synchronize()
        return h, dt, coarse_ms, dt_fused

    def measure_graph(Mg, reps):
        """Per-call µs of i2h_head replayed from a HIP graph that holds one call per cold copy (the
        library allocates, clears and synchronises nothing, so the whole call is captured); the
        first replay's outputs are checked against eager calls."""
        x = x_all[:Mg].contiguous()
        ws = torch.empty(i2h.workspace_bytes(Mg, N, K, KC, R), dtype=torch.uint8, device=dev)
        outs = [(torch.empty(Mg, 1, dtype=torch.int32, device=dev), torch.empty(Mg, 1, dtype=torch.float32, device=dev))
                for _ in copies]
        eager = [i2h.head(x, p_, S_, Z_, W, kcand=KC, R=R, k=1) for (p_, S_, Z_) in copies]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for (p_, S_, Z_), o in zip(copies, outs):
                i2h.head(x, p_, S_, Z_, W, kcand=KC, R=R, k=1, workspace=ws, out=o)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for (p_, S_, Z_), o in zip(copies, outs):
                i2h.head(x, p_, S_, Z_, W, kcand=KC, R=R, k=1, workspace=ws, out=o)
        for o in outs:
            o[0].fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for (ei, ev), (oi, ov) in zip(eager, outs):
            if not (torch.equal(ei, oi) and torch.equal(ev, ov)):
                raise RuntimeError("graph replay differs from the eager call")
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) * 1e3 / (reps * len(copies))

    def measure_fp8(h, steps, warmup):
        """The FP8 e4m3 per-row-scale source (the same weights in FP8): its load-time pack, and the
        fused tail (selection, exact rerank against the FP8 rows, argmax) beside the bf16 one, each
        timed back to back with HIP events on the candidates of one coarse call."""
        W8, wsc = si.fp8_head_of(W)
        pk8 = []
        p8 = i2h.pack_fp8(W8, wsc)
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            i2h.pack_fp8(W8, wsc, out=p8)
            b.record()
            torch.cuda.synchronize()
            pk8.append(a.elapsed_time(b) * 1e3)
        h.step(0)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        a_fp8 = (P(h.cs), P(h.ci), M, (N + 63) // 64, KC, R, P(h.x), P(W8), P(wsc), W8.stride(0), N, K, 1, None,
                 None, P(h.oi), P(h.ov), h.stream)

        def tail_us(fn, args_):
            return back_to_back_us(torch, lambda: fn(*args_), steps, warmup)

        L = h.lib
        res = dict(pack_us=round(float(np.median(pk8)), 1),
                   pack_bytes=N * K + 4 * N + N * K // 4 + 2 * N * (K // 128) * 2,
                   tail_fp8_us=round(tail_us(L.i2h_select_rerank_topk_fp8, a_fp8), 2),
                   tail_bf16_us=round(tail_us(L.i2h_select_rerank_topk, h.a_srr), 2))
        res["pack_gbps"] = round(res["pack_bytes"] / (res["pack_us"] * 1e-6) / 1e9, 1)
        del W8, wsc, p8
        torch.cuda.synchronize()
        return res

    def measure_int4(h, steps, warmup):
        """The int4 head (the page's comparison point) on the same weights at KCAND = 1: its pack,
        and per call xsum + int4 coarse + the fused tail, with the coarse kernel alone timed back
        to back on cold copies; argmax agreement with the int2 head's GPU call on the match rows."""
        p4 = i2h.pack4(W)
        pk4 = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            i2h.pack4(W, out=p4)
            b.record()
            torch.cuda.synchronize()
            pk4.append(a.elapsed_time(b) * 1e3)
        cps = [p4] + [(p4[0].clone(), p4[1].clone(), p4[2].clone()) for _ in range(5)]
        nblk = (N + 63) // 64
        x = h.x
        xs = torch.empty(M, K // 128, dtype=torch.float32, device=x.device)
        cs = torch.empty(M, nblk, dtype=torch.float32, device=x.device)
        ci = torch.empty(M, nblk, dtype=torch.int32, device=x.device)
        oi = torch.empty(M, 1, dtype=torch.int32, device=x.device)
        ov = torch.empty(M, 1, dtype=torch.float32, device=x.device)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        L = h.lib
        a_c = [(P(x), P(xs), M, P(p), P(S), P(Z), N, K, 1, P(cs), P(ci), None, h.stream) for (p, S, Z) in cps]
        a_t = (P(cs), P(ci), M, nblk, 1, R, P(x), P(W), W.stride(0), N, K, 1, None, None, P(oi), P(ov), h.stream)

        def call(i):
            st = L.i2h_xsum(P(x), M, K, P(xs), h.stream)
            st |= L.i2h_coarse4_topk(*a_c[i % len(a_c)])
            st |= L.i2h_select_rerank_topk(*a_t)
            if st:
                raise RuntimeError(f"libi2h status {st}")

        d, _ = time_steps(torch, call, steps, warmup)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(steps):
            L.i2h_coarse4_topk(*a_c[i % len(a_c)])
        ev1.record()
        torch.cuda.synchronize()
        c_us = ev0.elapsed_time(ev1) * 1e3 / steps
        cbytes = N * K // 2 + 4 * N * (K // 128) + M * K * 2 + M * (K // 128) * 4 + M * nblk * 8
        argmax4 = []
        for r in range(args.match_rows):
            xr = x_all[r:r + 1].contiguous()
            c4s, c4i = i2h.coarse4_topk(xr, i2h.xsum(xr), *p4, kcand=1)
            i4, _ = i2h.select_rerank_topk(c4s, c4i, 1, R, xr, W, 1)
            argmax4.append(int(i4.item()))
        del cps, p4
        torch.cuda.synchronize()
        return dict(kcand=1, us_per_call=round(d * 1e6, 2), coarse_us=round(c_us, 2), coarse_bytes=cbytes,
                    coarse_gbps=round(cbytes / (c_us * 1e-6) / 1e9, 1),
                    coarse_hbm_frac=round(cbytes / (c_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    pack_us=round(float(np.median(pk4)), 1), argmax_rows=argmax4)

    def measure_selection(h, steps, warmup):
        """Block candidates (the design) against a token-level top-R over the whole coarse row:
        per call, and the tail alone (selection + exact rerank + argmax) on one call's outputs."""
        L = h.lib
        d_tok, _ = time_steps(torch, h.token_level, steps, warmup)
        h.token_level(0)
        tail_tok = back_to_back_us(torch, lambda: L.i2h_select_tokens(*h.a_seltok) | L.i2h_rerank_topk(*h.a_rr_sel),
                                   steps, warmup)
        sel_tok = back_to_back_us(torch, lambda: L.i2h_select_tokens(*h.a_seltok), steps, warmup)
        h.step(0)
        tail_blk = back_to_back_us(torch, lambda: L.i2h_select_rerank_topk(*h.a_srr), steps, warmup)
        rows = []
        for r in range(args.match_rows):
            xr = x_all[r:r + 1].contiguous()
            _, _, yr = i2h.coarse_topk(xr, None if i2h.coarse_sums_x(1, K) else i2h.xsum(xr), packed, S, ZS,
                                       kcand=KC, want_y=True)
            ir, _ = i2h.rerank_topk(xr, W, i2h.select_tokens(yr, R), 1)
            rows.append(int(ir.item()))
        torch.cuda.synchronize()
        return dict(token_level_us_per_call=round(d_tok * 1e6, 2), token_level_tail_us=round(tail_tok, 2),
                    select_tokens_us=round(sel_tok, 2), block_tail_us=round(tail_blk, 2), argmax_rows=rows)

    def measure_variants(steps, warmup):
        """The design alternatives at the workload shape (one property changed each): each variant's
        load-time pack, and its coarse kernel alone at M = 1 and 16, back to back over cold copies,
        with the production coarse kernel's time beside them."""
        combos = (("design", 128, "quarter", "accumulator"), ("group64", 64, "quarter", "accumulator"),
                  ("contiguous4", 128, "contiguous", "accumulator"), ("weight_tile", 128, "quarter", "tile"))
        Pp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        L = i2h.lib()
        nblk = (N + 63) // 64
        res = {}
        for name, g, lay, sc in combos:
            pk = i2h.pack_variant(W, g, lay)
            torch.cuda.synchronize()
            t = []
            for _ in range(3):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                i2h.pack_variant(W, g, lay)
                b.record()
                torch.cuda.synchronize()
                t.append(a.elapsed_time(b) * 1e3)
            cps = [pk] + [tuple(u.clone() for u in pk) for _ in range(COPIES - 1)]
            r = dict(group=g, layout=lay, scaling=sc, pack_us=round(float(np.median(t)), 1),
                     weight_bytes=N * K // 4 + 2 * N * (K // g) * 2)
            for Mv in (1, 16):
                xv = x_all[:Mv].contiguous()
                xs = i2h.xsum_group(xv, g) if sc == "accumulator" else None
                cs = torch.empty(Mv, nblk * KC, dtype=torch.float32, device=dev)
                ci = torch.empty(Mv, nblk * KC, dtype=torch.int32, device=dev)
                lay_c, sc_c = (0 if lay == "quarter" else 1), (0 if sc == "accumulator" else 1)
                args_ = [(Pp(xv), Pp(xs), Mv, Pp(p), Pp(S_), Pp(Z_), N, K, g, lay_c, sc_c, KC, Pp(cs), Pp(ci), stream)
                         for (p, S_, Z_) in cps]
                it = iter(range(1 << 30))
                us = back_to_back_us(torch, lambda: L.i2h_coarse_variant_topk(*args_[next(it) % len(args_)]),
                                     steps, warmup)
                r[f"M{Mv}_coarse_us"] = round(us, 2)
                r[f"M{Mv}_hbm_frac"] = round((r["weight_bytes"] + Mv * K * 2) / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            res[name] = r
            del cps, pk
            torch.cuda.synchronize()
        for name in res:
            for Mv in (1, 16):
                res[name][f"M{Mv}_vs_design"] = round(res[name][f"M{Mv}_coarse_us"] / res["design"][f"M{Mv}_coarse_us"], 3)
        return res

    def measure_full_vocab(steps, warmup):
        """The unsharded 248320-row vocabulary with the top-16 caller: the GPU quantise+pack of the
        bf16 weight (2.54 GB) timed on its own, then one i2h_head call (top-16 drawn from the 32
        reranked tokens) at each M of the band list, on 6 rotated packed copies (2.1 GB)."""
        cfg = si.WORKLOADS["full_vocab_top16_k5120_n248320"]
        Nf, Kf, kf = cfg["N"], cfg["K"], cfg["topk"]
        Wf = si.gen_weight(Nf, Kf).to(dev)
        pf = i2h.pack(Wf)
        pk = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            i2h.pack(Wf, out=pf)
            b.record()
            torch.cuda.synchronize()
            pk.append(a.elapsed_time(b) * 1e3)
        pbytes = Nf * Kf * 2 + Nf * Kf // 4 + 2 * Nf * (Kf // 128) * 2
        cps = [pf] + [(pf[0].clone(), pf[1].clone(), pf[2].clone()) for _ in range(5)]
        xf = si.gen_x(max(cfg["M"]), Kf, outliers=cfg["outliers"]).to(dev)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        s = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        L = i2h.lib()
        rows = []
        for Mf in cfg["M"]:
            x = xf[:Mf].contiguous()
            oi = torch.empty(Mf, kf, dtype=torch.int32, device=dev)
            ov = torch.empty(Mf, kf, dtype=torch.float32, device=dev)
            wsn = i2h.workspace_bytes(Mf, Nf, Kf, KC, R)
            ws = torch.empty(max(wsn, 1), dtype=torch.uint8, device=dev)
            args = [(P(x), Mf, P(p), P(S_), P(Z_), P(Wf), Wf.stride(0), Nf, Kf, KC, R, kf, P(oi), P(ov), None,
                     P(ws), wsn, s) for (p, S_, Z_) in cps]
            it = iter(range(1 << 30))
            us_f = back_to_back_us(torch, lambda: L.i2h_head(*args[next(it) % len(args)]), steps, warmup)
            hb_f = head_bytes(Mf, Nf, Kf, k=kf, own_sums=i2h.coarse_sums_x(Mf, Kf))
            fl = 2.0 * Mf * Kf * Nf
            rows.append(dict(M=Mf, us_per_call=round(us_f, 2), gbps=round(hb_f["total"] / us_f / 1e3, 1),
                             hbm_frac=round(hb_f["total"] / us_f / 1e3 / HBM_PEAK_GBS, 4),
                             tflops_useful=round(fl / us_f / 1e6, 1),
                             mfma_util_useful=round(fl / us_f / 1e6 / BF16_PEAK_TFS, 4)))
        res = dict(N=Nf, K=Kf, topk=kf, cold_cache_copies=len(cps),
                   pack_us=round(float(np.median(pk)), 1),
                   pack_gbps=round(pbytes / (float(np.median(pk)) * 1e-6) / 1e9, 1),
                   pack_hbm_frac=round(pbytes / (float(np.median(pk)) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   calls=rows)
        del Wf, pf, cps
        torch.cuda.synchronize()
        return res

    def measure_dropin(h, steps, warmup):
        """The drop-in logits row (argmax and top-k callers): per-call time and the write-back alone."""
        res = {}
        for topk in (False, True):
            d, _ = time_steps(torch, lambda i, t=topk: h.dropin(i, t), steps, warmup)
            h.logits_only(torch, warmup, topk)
            lu = h.logits_only(torch, steps, topk)
            name = "topk" if topk else "argmax"
            res[f"{name}_us_per_call"] = round(d * 1e6, 2)
            res[f"{name}_logits_us"] = round(lu, 2)
        torch.cuda.synchronize()
        return res

    log(f"[bench] timing M={M}: {args.warmup} warmup + {args.steps} steps")
    h, dt, coarse_ms, dt_fused = measure(M, args.steps, args.warmup, PREWARM_S)
    hb = head_bytes(M, N, K, own_sums=h.own_sums)
    pct = call_percentiles(torch, np, h.fused, args.steps, args.warmup + args.steps)
    log(f"[bench] i2h_head replayed from a HIP graph at M={M}")
    us_graph = measure_graph(M, max(10, args.steps // 12))
    us = dt * 1e6
    coarse_us = coarse_ms * 1e3
    achieved = hb["coarse"] / (coarse_us * 1e-6) / 1e9
    traffic = traffic_for(M)
    log(f"[bench] FP8 weight source at M={M}: pack and fused tail")
    fp8 = measure_fp8(h, args.steps, args.warmup)
    log(f"[bench] int4 head at M={M}, KCAND=1: pack, coarse and per call")
    int4 = measure_int4(h, args.steps, args.warmup)
    log(f"[bench] selection: block candidates against token-level top-{R} at M={M}")
    selab = measure_selection(h, args.steps, args.warmup)
    selab["block_us_per_call"] = round(us, 2)
    log("[bench] design alternatives: group 64, contiguous-4 bytes, dequantised weight tile")
    variants = measure_variants(args.steps, args.warmup)
    log(f"[bench] timing the drop-in logits row at M={M}")
    dropin = measure_dropin(h, args.steps, args.warmup)
    dropin["logits_bytes"] = {"argmax": M * N * 2 * 2 + M * R * 8, "topk": M * N * 2 + M * R * 8}

    full_vocab = None
    if not args.no_bands:
        log("[bench] full vocabulary (248320 rows), top-16 caller: pack and one call per M")
        full_vocab = measure_full_vocab(max(20, args.steps // 4), max(5, args.warmup // 2))

    bands = []
    if not args.no_bands:
        for Mb in (16, 32, 64):
            log(f"[bench] timing band M={Mb}")
            hbh, dtb, cmsb, dtfb = measure(Mb, max(20, args.steps // 2), max(5, args.warmup // 2))
            hbb = head_bytes(Mb, N, K, own_sums=hbh.own_sums)
            flops = 2.0 * Mb * K * N
            bands.append(dict(M=Mb, us_per_call=round(dtfb * 1e6, 2),
                              us_per_call_separate_entries=round(dtb * 1e6, 2),
                              us_per_call_graph=round(measure_graph(Mb, max(10, args.steps // 24)), 2),
                              coarse_us=round(cmsb * 1e3, 2),
                              gbps=round(hbb["total"] / dtfb / 1e9, 1),
                              coarse_gbps=round(hbb["coarse"] / (cmsb * 1e-3) / 1e9, 1),
                              coarse_hbm_frac=round(hbb["coarse"] / (cmsb * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              coarse_tflops_useful=round(flops / (cmsb * 1e-3) / 1e12, 2),
                              mfma_util_useful=round(flops / (cmsb * 1e-3) / 1e12 / BF16_PEAK_TFS, 4),
                              coarse_traffic_bytes=traffic_for(Mb)))

    # argmax match against the oracle on the first rows, one call per row as in the timed step
    result = {}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log(f"[bench] argmax match on {args.match_rows} rows (GPU calls of M=1)")
        got = []
        for r in range(args.match_rows):
            idx, _ = i2h.head(x_all[r:r + 1].contiguous(), packed, S, ZS, W, kcand=KC, R=R, k=1)
            got.append(int(idx.item()))
        Wb, xb = si.bits(Wc), si.bits(x_all_c[:args.match_rows])
        log("[bench] oracle pack (untimed, load-time step)")
        po, So, ZSo = oracle.pack(Wb)
        threads = oracle.int2_head._threads()
        log("[bench] oracle head, one call of the timed workload (timed)")
        t0 = time.perf_counter()
        r1 = oracle.head(xb[:1], Wb, po, So, ZSo, kcand=KC, R=R, k=1)
        cpu_s = time.perf_counter() - t0
        log("[bench] oracle head on the match rows")
        ro = oracle.head(xb, Wb, po, So, ZSo, kcand=KC, R=R, k=1)
        want = [int(v) for v in ro["idx"][:, 0]]
        match = sum(int(a == b) for a, b in zip(got, want))
        ex = oracle.exact_logits(xb, Wb)
        recall = sum(int(a == b) for a, b in zip(want, ex.argmax(1)))
        dense = ex.argmax(1)
        result = dict(argmax_match_pct=round(100.0 * match / len(want), 2), argmax_rows=len(want),
                      recall_vs_dense_bf16_pct=round(100.0 * recall / len(want), 2))
        selab["token_level_recall_vs_dense_bf16_pct"] = round(
            100.0 * sum(int(a == b) for a, b in zip(selab["argmax_rows"], dense)) / len(want), 2)
        int4["recall_vs_dense_bf16_pct"] = round(
            100.0 * sum(int(a == b) for a, b in zip(int4["argmax_rows"], dense)) / len(want), 2)
        assert int(r1["idx"][0, 0]) == want[0]
        cpu = dict(value=round(hb["total"] / cpu_s / 1e9, 4), unit="GB/s", us_per_call=round(cpu_s * 1e6, 1),
                   cores=threads, kind="oracle",
                   sample=f"one call of the {WORKLOAD} head (coarse over all {N} rows, emit, select, rerank, "
                          f"argmax) on the numpy oracle with {threads} threads; pack excluded")

    out = {
        "metric": METRIC,
        "value": round(hb["total"] / dt_fused / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt_fused * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "M": M, "K": K, "N": N, "kcand": KC, "R": R, "output": "argmax",
                   "cold_cache_copies": COPIES, "group": 128, "block_n": 64},
        "us_per_call": round(dt_fused * 1e6, 2),
        "us_per_call_separate_entries": round(us, 2),
        "us_per_call_graph": round(us_graph, 2),
        "us_per_call_p10_p50_p90": pct,
        "bytes_per_call": hb["total"],
        "gbps_packed_only": round(N * K / 4 / dt_fused / 1e9, 1),
        "hbm_frac": round(hb["total"] / dt_fused / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "copy_gbps_measured": copy_gbps(torch, dev),
                     "kernel": "coarse_small_kernel<1, true, 10>", "kernel_us": round(coarse_us, 2),
                     "algorithmic_bytes": hb["coarse"]},
        "pack": {"us": round(pack_us, 1), "gbps": round(pack_bytes / (pack_us * 1e-6) / 1e9, 1),
                 "hbm_frac": round(pack_bytes / (pack_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "N": N, "K": K},
        "dropin_logits": dropin,
        "fp8_source": fp8,
        "int4_head": {k_: v_ for k_, v_ in int4.items() if k_ != "argmax_rows"},
        "ablations": {"selection": {k_: v_ for k_, v_ in selab.items() if k_ != "argmax_rows"},
                      "coarse_variants": variants},
        **result,
        "bands": bands,
        "full_vocab_top16": full_vocab,
        "device": device_info(torch),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
