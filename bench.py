"""Benchmark of the int2 draft LM head on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-bands]
    python bench.py --traffic-probe    # short run for rocprofv3 counter passes (see below)
    python bench.py --variant-probe    # the same for the design alternatives

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
`ablations.coarse_variants` times the production coarse kernels in four forms that differ in one
property each (the design itself: group 128, quarter-split, scale on the accumulator; group 64;
contiguous-4 bytes; dequantised weight tile) at M = 1 (the one-row kernel) and 16 (the 16-row
tile), group sums taken in the kernel as the head does, on cold copies, with each pack.
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


COARSE_SOURCES = ("coarse.hip", "coarse_tile.hip", "ablation.h", "dequant.h", "device_util.h", "block_emit.h")


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


def variant_probe(torch, i2h, si, dev):
    """Launches for rocprofv3 counter passes over the design alternatives: each of the four forms
    (design, group 64, contiguous-4, weight tile) packed from the timed workload's weight, then its
    coarse kernel at M = 1 and 16 on 4 cold copies, 6 launches each; then the plain 512 MiB device
    copy of traffic_probe (4 launches) that calibrates the byte counters."""
    cfg = si.WORKLOADS[WORKLOAD]
    K, N = cfg["K"], cfg["N"]
    W = si.gen_weight(N, K).to(dev)
    x_all = si.gen_x(16, K, outliers=cfg["outliers"]).to(dev)
    combos = ((128, "quarter", "accumulator"), (64, "quarter", "accumulator"), (128, "contiguous", "accumulator"),
              (128, "quarter", "tile"))
    for g, lay, sc in combos:
        pk = i2h.pack_variant(W, g, lay)
        cps = [pk] + [tuple(u.clone() for u in pk) for _ in range(3)]
        for M in (1, 16):
            x = x_all[:M].contiguous()
            for i in range(6):
                p, a, b = cps[i % 4]
                i2h.coarse_variant_topk(x, None, p, a, b, g, lay, sc, KC)
            torch.cuda.synchronize()
        del cps, pk
    src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"variant_probe": True, "M": [1, 16], "copy_bytes": src.numel()}), flush=True)


# Windows within which a final place that differs from the oracle's is excused: two reranked tokens
# whose exact scores (fp64) tie within EXACT_TIE, or a selected set that differs from the oracle's
# only by tokens whose coarse scores lie within COARSE_TIE * max|c| of the oracle's R-th best. The
# tight windows are counted beside them.
EXACT_TIE, EXACT_TIE_TIGHT = 1e-3, 1e-5
COARSE_TIE, COARSE_TIE_TIGHT = 2e-3, 1e-4


def gpu_batches(i2h, torch, np, x, packed, S, ZS, W, M, k):
    """(idx [rows, k], sel [rows, R]) for the rows of x in calls of M rows: i2h_head's answer, and
    the selection from the same kernels called through their entry points (the coarse pass and the
    fused tail with its selection), whose answer must equal i2h_head's."""
    K = x.shape[1]
    idx, sel = [], []
    for r0 in range(0, x.shape[0], M):
        xb = x[r0:r0 + M].contiguous()
        hi, _ = i2h.head(xb, packed, S, ZS, W, kcand=KC, R=R, k=k)
        xs = None if i2h.coarse_sums_x(xb.shape[0], K) else i2h.xsum(xb)
        cs, ci, _ = i2h.coarse_topk(xb, xs, packed, S, ZS, kcand=KC)
        oi, _, sl, _ = i2h.select_rerank_topk(cs, ci, KC, R, xb, W, k, want_sel=True)
        if not torch.equal(hi, oi):
            raise RuntimeError("i2h_head differs from its kernels called through their entry points")
        idx.append(hi.cpu().numpy())
        sel.append(sl.cpu().numpy())
    return np.concatenate(idx), np.concatenate(sel)


def classify(oracle, np, gpu_idx, gpu_sel, res, xb, Wb):
    """Final places of the GPU against the oracle's: equal, excused (an exact-score tie inside an
    equal selection, or a selection that differs at its edge), or unexcused."""
    c, so, io = res["coarse"], res["sel"], res["idx"]
    rows, k = gpu_idx.shape
    scale = np.abs(c).max(axis=1)
    n = dict(rows=int(rows), places=int(rows * k), match=0, exact_tie=0, exact_tie_tight=0, selection_edge=0,
             selection_edge_tight=0, unexcused=0)
    for m in range(rows):
        go = set(int(t) for t in gpu_sel[m] if t >= 0)
        oo = set(int(t) for t in so[m] if t >= 0)
        for j in range(k):
            a, b = int(gpu_idx[m, j]), int(io[m, j])
            if a == b:
                n["match"] += 1
                continue
            if go == oo:
                e = oracle.rerank_exact(xb[m:m + 1], Wb, np.array([[a, b]], np.int32))[0]
                gap = abs(e[0] - e[1])
                key, tight = ("exact_tie", gap <= EXACT_TIE_TIGHT) if gap <= EXACT_TIE else (None, False)
            else:
                thr = c[m, so[m][len(oo) - 1]]
                gap = max(abs(c[m, t] - thr) for t in go ^ oo) / scale[m]
                key, tight = ("selection_edge", gap <= COARSE_TIE_TIGHT) if gap <= COARSE_TIE else (None, False)
            if key is None:
                n["unexcused"] += 1
            else:
                n[key] += 1
                n[key + "_tight"] += int(tight)
    n["match_pct"] = round(100.0 * n["match"] / n["places"], 3)
    n["match_or_excused_pct"] = round(100.0 * (n["places"] - n["unexcused"]) / n["places"], 3)
    return n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bands", action="store_true")
    ap.add_argument("--variant-probe", action="store_true",
                    help="launch each design alternative at M = 1 and 16 (for rocprofv3 counter passes) and exit")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only launch the coarse kernel 6 times per M in (1, 16, 32, 64) on cold weight copies, "
                         "then copy a 512 MiB buffer 4 times (the calibration kernel for HBM byte counters)")
    ap.add_argument("--match-rows", type=int, default=1024,
                    help="rows of x compared with the oracle at M = 1, 16 and 64 (and the tiny head)")
    ap.add_argument("--match-rows-full-vocab", type=int, default=128,
                    help="rows of x compared with the oracle on the full vocabulary (top-16, calls of 16 rows)")
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
    if args.variant_probe:
        variant_probe(torch, i2h, si, dev)
        return
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
    x_all_c = si.gen_x(nrows, K, outliers=cfg["outliers"])  # the match rows (and the timed batches' rows)
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
                xs = None  # group sums taken in the kernel, as the head's calls do
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
        Wf_c = si.gen_weight(Nf, Kf)
        Wf = Wf_c.to(dev)
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
        xf_c = si.gen_x(max(max(cfg["M"]), args.match_rows_full_vocab), Kf, outliers=cfg["outliers"])
        xf = xf_c.to(dev)
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
            a_head = [(P(x), Mf, P(p), P(S_), P(Z_), P(Wf), Wf.stride(0), Nf, Kf, KC, R, kf, P(oi), P(ov), None,
                       P(ws), wsn, s) for (p, S_, Z_) in cps]
            it = iter(range(1 << 30))
            us_f = back_to_back_us(torch, lambda: L.i2h_head(*a_head[next(it) % len(a_head)]), steps, warmup)
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
        match = None
        if not args.no_cpu_baseline:
            # top-16 of the match rows in calls of 16 rows, for the comparison with the oracle
            gi, gs = gpu_batches(i2h, torch, np, xf[:args.match_rows_full_vocab], *pf, Wf, 16, kf)
            match = dict(W=Wf_c, x=xf_c[:args.match_rows_full_vocab], idx=gi, sel=gs, k=kf)
        del Wf, pf, cps
        torch.cuda.synchronize()
        return res, match

    def measure_tiny(steps, warmup):
        """The tiny head (M = 1, K = 512, N = 4096; 0.63 MB, resident in L2): i2h_head per call back
        to back, the spread over single calls, and the GPU answers on the match rows."""
        cfg = si.WORKLOADS["tiny_head_m1_k512_n4096"]
        Nt, Kt = cfg["N"], cfg["K"]
        Wt_c = si.gen_weight(Nt, Kt)
        xt_c = si.gen_x(max(args.match_rows, 1), Kt, outliers=cfg["outliers"])
        Wt, xt = Wt_c.to(dev), xt_c.to(dev)
        pt = i2h.pack(Wt)
        x1 = xt[:1].contiguous()
        wsn = i2h.workspace_bytes(1, Nt, Kt, KC, R)
        ws = torch.empty(wsn, dtype=torch.uint8, device=dev)
        oi = torch.empty(1, 1, dtype=torch.int32, device=dev)
        ov = torch.empty(1, 1, dtype=torch.float32, device=dev)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        s_ = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        a = (P(x1), 1, P(pt[0]), P(pt[1]), P(pt[2]), P(Wt), Wt.stride(0), Nt, Kt, KC, R, 1, P(oi), P(ov), None,
             P(ws), wsn, s_)
        L = i2h.lib()
        us_t = back_to_back_us(torch, lambda: L.i2h_head(*a), steps, warmup)
        pct_t = call_percentiles(torch, np, lambda i: L.i2h_head(*a), steps, warmup)
        hb_t = head_bytes(1, Nt, Kt, own_sums=i2h.coarse_sums_x(1, Kt))
        res = dict(workload="tiny_head_m1_k512_n4096", M=1, K=Kt, N=Nt, us_per_call=round(us_t, 2),
                   us_per_call_p10_p50_p90=pct_t, bytes_per_call=hb_t["total"],
                   note="0.63 MB of algorithmic bytes stay in L2: a latency figure, not a bandwidth one")
        match = None
        if not args.no_cpu_baseline:
            gi, gs = gpu_batches(i2h, torch, np, xt[:args.match_rows], *pt, Wt, 1, 1)
            match = dict(W=Wt_c, x=xt_c[:args.match_rows], idx=gi, sel=gs, k=1)
        return res, match

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

    log("[bench] tiny head (M=1, K=512, N=4096)")
    tiny, tiny_match = measure_tiny(args.steps, args.warmup)

    full_vocab, fv_match = None, None
    if not args.no_bands:
        log("[bench] full vocabulary (248320 rows), top-16 caller: pack and one call per M")
        full_vocab, fv_match = measure_full_vocab(max(20, args.steps // 4), max(5, args.warmup // 2))

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
                              gbps_packed_only=round(N * K / 4 / dtfb / 1e9, 1),
                              hbm_frac=round(hbb["total"] / dtfb / 1e9 / HBM_PEAK_GBS, 4),
                              coarse_gbps=round(hbb["coarse"] / (cmsb * 1e-3) / 1e9, 1),
                              coarse_gbps_packed_only=round(N * K / 4 / (cmsb * 1e-3) / 1e9, 1),
                              coarse_hbm_frac=round(hbb["coarse"] / (cmsb * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              coarse_tflops_useful=round(flops / (cmsb * 1e-3) / 1e12, 2),
                              mfma_util_useful=round(flops / (cmsb * 1e-3) / 1e12 / BF16_PEAK_TFS, 4),
                              coarse_traffic_bytes=traffic_for(Mb), group_sums_in_kernel=hbh.own_sums))

    # The CPU leg: the oracle timed on the host cores, and the GPU answers compared with the
    # oracle's on every configuration (the tiny head; the draft slot at M = 1, 16, 64 on the same
    # rows; the full vocabulary's top-16)
    result = {}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log(f"[bench] GPU answers on {args.match_rows} rows in calls of 1, 16 and 64 rows")
        xm = x_all[:args.match_rows]
        gpu_rows = {Mb: gpu_batches(i2h, torch, np, xm, packed, S, ZS, W, Mb, 1) for Mb in (1, 16, 64)}
        Wb, xb = si.bits(Wc), si.bits(x_all_c[:args.match_rows])
        threads = oracle.int2_head._threads()
        try:
            affinity = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            affinity = os.cpu_count() or 1
        log("[bench] oracle pack (untimed, load-time step)")
        po, So, ZSo = oracle.pack(Wb)
        log("[bench] oracle head, single calls of the timed workload (timed, median of 5)")
        ts_ = []
        for r in range(5):
            t0 = time.perf_counter()
            r1 = oracle.head(xb[r:r + 1], Wb, po, So, ZSo, kcand=KC, R=R, k=1)
            ts_.append(time.perf_counter() - t0)
        cpu_s = float(np.median(ts_))
        log(f"[bench] oracle head on the {args.match_rows} match rows")
        ro = oracle.head(xb, Wb, po, So, ZSo, kcand=KC, R=R, k=1)
        assert int(r1["idx"][0, 0]) == int(ro["idx"][4, 0])
        match = {}
        for Mb, name in ((1, "draft_slot_m1"), (16, "draft_band_m16"), (64, "draft_band_m64")):
            match[name] = classify(oracle, np, gpu_rows[Mb][0], gpu_rows[Mb][1], ro, xb, Wb)
        want = ro["idx"][:, 0]
        dense = oracle.exact_logits(xb, Wb).argmax(1)
        recall = int((want == dense).sum())
        log("[bench] oracle on the tiny head")
        po_t = oracle.pack(si.bits(tiny_match["W"]))
        xtb = si.bits(tiny_match["x"])
        rt = oracle.head(xtb, si.bits(tiny_match["W"]), *po_t, kcand=KC, R=R, k=1)
        match["tiny_head_m1"] = classify(oracle, np, tiny_match["idx"], tiny_match["sel"], rt, xtb,
                                         si.bits(tiny_match["W"]))
        if fv_match is not None:
            log(f"[bench] oracle on the full vocabulary, {fv_match['x'].shape[0]} rows (top-16)")
            Wfb, xfb = si.bits(fv_match["W"]), si.bits(fv_match["x"])
            rf = oracle.head(xfb, Wfb, *oracle.pack(Wfb), kcand=KC, R=R, k=fv_match["k"])
            match["full_vocab_top16_m16"] = classify(oracle, np, fv_match["idx"], fv_match["sel"], rf, xfb, Wfb)
            del Wfb, rf
        result = dict(argmax_match_pct=match["draft_slot_m1"]["match_pct"], argmax_rows=len(want),
                      argmax_match=match,
                      argmax_match_windows=dict(exact_tie=EXACT_TIE, exact_tie_tight=EXACT_TIE_TIGHT,
                                                selection_edge=COARSE_TIE, selection_edge_tight=COARSE_TIE_TIGHT),
                      recall_vs_dense_bf16_pct=round(100.0 * recall / len(want), 2))
        nr = min(len(want), len(selab["argmax_rows"]))
        selab["token_level_recall_vs_dense_bf16_pct"] = round(
            100.0 * sum(int(a == b) for a, b in zip(selab["argmax_rows"][:nr], dense[:nr])) / nr, 2)
        int4["recall_vs_dense_bf16_pct"] = round(
            100.0 * sum(int(a == b) for a, b in zip(int4["argmax_rows"][:nr], dense[:nr])) / nr, 2)
        cpu = dict(value=round(hb["total"] / cpu_s / 1e9, 4), unit="GB/s", us_per_call=round(cpu_s * 1e6, 1),
                   cores=threads, affinity_cores=affinity, kind="oracle",
                   sample=f"5 single-row calls of the {WORKLOAD} head (coarse over all {N} rows, emit, select, "
                          f"rerank, argmax) on the numpy oracle with {threads} threads, median; pack excluded")

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
                     "kernel": "coarse_small_kernel<1, true, 10, 0>", "kernel_us": round(coarse_us, 2),
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
        "tiny_head": tiny,
        "device": device_info(torch),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
