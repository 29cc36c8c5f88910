"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status codes before enqueuing anything. No call
here reaches a kernel launch, so these run without a GPU."""
import ctypes
import os
import re

import pytest

import bit_quantized_lm_int2_amd as i2h

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "i2h.h")

OK, ARG, SHAPE, ALIGN, LIMIT, WS = 0, -1, -2, -3, -4, -5
P = 0x10000          # a 64 KiB-aligned fake device address; never dereferenced on these paths
ODD = 0x10001


def declared():
    text = open(HEADER).read()
    return re.findall(r"I2H_API\s+[\w\s\*]+?\b(i2h_\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = set(declared())
    want = {"i2h_version", "i2h_strerror", "i2h_last_hip_error", "i2h_sizes", "i2h_pack", "i2h_xsum",
            "i2h_coarse_topk", "i2h_select", "i2h_rerank", "i2h_finalize", "i2h_workspace_bytes",
            "i2h_head", "i2h_head_noalloc", "i2h_coarse_sums_x", "i2h_rerank_topk",
            "i2h_select_rerank_topk", "i2h_logits", "i2h_pack_fp8", "i2h_rerank_fp8",
            "i2h_select_rerank_topk_fp8", "i2h_pack4", "i2h_coarse4_topk",
            "i2h_select_tokens", "i2h_select_tokens_workspace_bytes", "i2h_pack_variant", "i2h_xsum_group", "i2h_coarse_variant_topk"}
    assert names == want


def test_library_exports_every_declared_symbol():
    lib = i2h.lib()
    for name in declared():
        assert hasattr(lib, name), name
    assert lib.i2h_version() >= 100


def test_strerror_and_last_error():
    lib = i2h.lib()
    for code in (OK, ARG, SHAPE, ALIGN, LIMIT, WS, -6, -7, -8, -99):
        assert lib.i2h_strerror(code)
    assert lib.i2h_strerror(-7) != lib.i2h_strerror(-99)
    assert lib.i2h_last_hip_error() == 0


def test_sizes():
    assert i2h.sizes(124160, 5120) == (158_924_800, 4_966_400)
    assert i2h.sizes(4096, 512) == (4096 * 128, 4096 * 4)
    lib = i2h.lib()
    a, b = ctypes.c_int64(), ctypes.c_int64()
    assert lib.i2h_sizes(10, 640, ctypes.byref(a), ctypes.byref(b)) == SHAPE
    assert lib.i2h_sizes(0, 512, ctypes.byref(a), ctypes.byref(b)) == SHAPE
    assert lib.i2h_sizes(10, 512, None, ctypes.byref(b)) == ARG


def test_coarse_sums_x():
    lib = i2h.lib()
    assert lib.i2h_coarse_sums_x(1, 5120) == 1
    assert lib.i2h_coarse_sums_x(1, 1024) == 1
    assert lib.i2h_coarse_sums_x(3, 1536) == 1    # no tile kernel for this K: the small kernel
    assert lib.i2h_coarse_sums_x(3, 4096) == 1    # 2..32 rows: the 16- and 32-row tiles sum x themselves
    assert lib.i2h_coarse_sums_x(2, 512) == 1
    assert lib.i2h_coarse_sums_x(16, 5120) == 1
    assert lib.i2h_coarse_sums_x(32, 5120) == 1
    assert lib.i2h_coarse_sums_x(33, 5120) == 0   # the 64-row tile takes the sums from i2h_xsum
    assert lib.i2h_coarse_sums_x(64, 5120) == 0
    assert lib.i2h_coarse_sums_x(65, 5120) == 0   # chunks of 64 and 1 rows
    assert lib.i2h_coarse_sums_x(130, 512) == 0   # chunks of 64, 64 and 2 rows
    assert lib.i2h_coarse_sums_x(5, 1536) == 0    # no tile for this K and more than 4 rows
    assert lib.i2h_coarse_sums_x(4, 16384) == 0   # x does not fit in LDS
    assert lib.i2h_coarse_sums_x(1, 1000) == 0
    c = lib.i2h_coarse_topk
    assert c(P, None, 40, P, P, P, 4096, 1024, 8, P, P, None, None) == ARG  # xs required here
    assert c(P, None, 16, P, P, P, 4096, 1536, 8, P, P, None, None) == ARG  # generic kernel: xs required
    r = lib.i2h_rerank_topk
    assert r(P, 1, P, 512, 4096, 512, P, 32, 33, None, P, P, None) == LIMIT
    assert r(P, 1, P, 512, 4096, 512, P, 65, 1, None, P, P, None) == ARG     # exact needed for R > 64
    assert r(P, 1, None, 512, 4096, 512, P, 32, 1, None, P, P, None) == ARG


def test_workspace_bytes():
    lib = i2h.lib()
    n = lib.i2h_workspace_bytes(16, 124160, 5120, 8, 32)
    # xs + candidates (score + index) + sel + exact, each rounded up to 256 bytes
    assert n >= 16 * 40 * 4 + 2 * 16 * 1940 * 8 * 4 + 2 * 16 * 32 * 4
    assert n % 256 == 0
    assert lib.i2h_workspace_bytes(16, 124160, 5000, 8, 32) == SHAPE
    assert lib.i2h_workspace_bytes(16, 124160, 5120, 0, 32) == LIMIT
    assert lib.i2h_workspace_bytes(16, 124160, 5120, 8, 2000) == LIMIT
    assert lib.i2h_workspace_bytes(16, 64 * 8193, 5120, 8, 32) == SHAPE


def test_pack_rejections():
    lib = i2h.lib()
    assert lib.i2h_pack(None, 512, 4, 512, P, P, P, None) == ARG
    assert lib.i2h_pack(P, 512, 4, 500, P, P, P, None) == SHAPE
    assert lib.i2h_pack(P, 256, 4, 512, P, P, P, None) == SHAPE      # ldw < K
    assert lib.i2h_pack(P, 516, 4, 512, P, P, P, None) == ALIGN      # ldw % 8
    assert lib.i2h_pack(ODD + 1, 512, 4, 512, P, P, P, None) == ALIGN
    assert lib.i2h_pack(P, 512, 0, 512, P, P, P, None) == SHAPE


def test_coarse_select_rerank_finalize_rejections():
    lib = i2h.lib()
    c = lib.i2h_coarse_topk
    assert c(None, P, 1, P, P, P, 4096, 512, 8, P, P, None, None) == ARG
    assert c(P, P, 0, P, P, P, 4096, 512, 8, P, P, None, None) == SHAPE
    assert c(P, P, 1, P, P, P, 4096, 768, 8, P, P, None, None) == SHAPE
    assert c(P, P, 1, P, P, P, 4096, 512, 0, P, P, None, None) == LIMIT
    assert c(P, P, 1, P, P, P, 4096, 512, 65, P, P, None, None) == LIMIT
    assert c(P + 8, P, 1, P, P, P, 4096, 512, 8, P, P, None, None) == ALIGN
    assert c(P, P, 1, P, P, P, 4096, 512, 8, P, P, ODD, None) == ALIGN
    s = lib.i2h_select
    assert s(P, P, 1, 64, 8, 0, P, None) == LIMIT
    assert s(P, P, 1, 64, 8, 1025, P, None) == LIMIT
    assert s(P, P, 1, 64, 64, 256, P, None) == LIMIT               # R * kcand > 8192
    assert s(P, P, 1, 8193, 8, 32, P, None) == SHAPE
    assert s(P, P, 1, 64, 8, 32, None, None) == ARG
    r = lib.i2h_rerank
    assert r(P, 1, P, 512, 4096, 512, P, 0, P, None) == LIMIT
    assert r(P, 1, P, 500, 4096, 512, P, 32, P, None) == SHAPE
    assert r(P, 1, P, 516, 4096, 512, P, 32, P, None) == ALIGN
    assert r(P, 1, None, 512, 4096, 512, P, 32, P, None) == ARG
    f = lib.i2h_finalize
    assert f(P, P, 1, 32, 33, P, P, None) == LIMIT
    assert f(P, P, 1, 32, 0, P, P, None) == LIMIT
    assert f(P, P, 0, 32, 1, P, P, None) == SHAPE
    assert f(P, P, 1, 32, 1, P + 2, P, None) == ALIGN
    x = lib.i2h_xsum
    assert x(P, 1, 1000, P, None) == SHAPE
    assert x(P + 4, 1, 512, P, None) == ALIGN


def test_head_rejections():
    lib = i2h.lib()
    h = lib.i2h_head
    need = lib.i2h_workspace_bytes(1, 4096, 512, 8, 32)
    args = [P, 1, P, P, P, P, 512, 4096, 512, 8, 32, 1, P, P, None, P, need, None]

    def call(**kw):
        a = list(args)
        names = ["x", "M", "packed", "S", "ZS", "W", "ldw", "N", "K", "kcand", "R", "k", "oi", "ov",
                 "y", "ws", "wsb", "stream"]
        for k_, v in kw.items():
            a[names.index(k_)] = v
        return h(*a)

    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(ws=P + 16) == ALIGN
    assert call(k=33) == LIMIT
    assert call(kcand=64, R=256, wsb=1 << 40) == LIMIT
    assert call(K=640) == SHAPE
    assert call(W=None) == ARG
    assert call(ldw=256) == SHAPE


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(i2h, "_lib", None)
    monkeypatch.setattr(i2h, "_LIB_PATH", "/nonexistent/libi2h.so")
    with pytest.raises(ImportError):
        i2h.lib()


def test_select_rerank_rejects_before_launch():
    f = i2h.lib().i2h_select_rerank_topk
    # cand_score, cand_idx, M, nblk, kcand, R, x, W, ldw, N, K, k, sel, exact, out_idx, out_val, stream
    assert f(None, P, 1, 1940, 8, 32, P, P, 5120, 124160, 5120, 1, None, None, P, P, None) == ARG
    assert f(P, P, 1, 1939, 8, 32, P, P, 5120, 124160, 5120, 1, None, None, P, P, None) == SHAPE  # nblk != ceil(N/64)
    assert f(P, P, 1, 1940, 8, 32, P, P, 5000, 124160, 5120, 1, None, None, P, P, None) == SHAPE  # ldw < K
    assert f(P, P, 1, 1940, 9, 32, P, P, 5120, 124160, 5120, 1, None, None, P, P, None) == LIMIT  # kcand > 8
    assert f(P, P, 1, 1940, 8, 65, P, P, 5120, 124160, 5120, 1, None, None, P, P, None) == LIMIT  # R > 64
    assert f(P, P, 1, 1940, 8, 32, P, P, 5120, 124160, 5120, 33, None, None, P, P, None) == LIMIT  # k > R
    assert f(P, P, 1, 4097, 8, 32, P, P, 5120, 262145, 5120, 1, None, None, P, P, None) == LIMIT  # N too large
    assert f(P, P, 1, 1940, 8, 32, P, P, 5124, 124160, 5120, 1, None, None, P, P, None) == ALIGN  # ldw % 8


def test_logits_rejects_before_launch():
    f = i2h.lib().i2h_logits
    BF, F16, F32 = 1, 2, 3
    # y, M, N, sel, exact, R, topk_only, bias, bias_dtype, out, out_dtype, stream
    assert f(None, 1, 124160, P, P, 32, 0, None, 0, P, BF, None) == ARG        # y needed for an argmax caller
    assert f(P, 1, 124160, P, P, 32, 0, None, 0, None, BF, None) == ARG        # no out
    assert f(P, 1, 124160, P, P, 32, 0, None, BF, P, BF, None) == ARG          # bias dtype without bias
    assert f(P, 1, 124160, P, P, 32, 0, P, 0, P, BF, None) == ARG              # bias without dtype
    assert f(P, 1, 124160, P, P, 32, 0, None, 0, P, 0, None) == ARG            # no out dtype
    assert f(P, 1, 124160, P, P, 32, 0, None, 0, P, 4, None) == ARG
    assert f(P, 0, 124160, P, P, 32, 0, None, 0, P, BF, None) == SHAPE
    assert f(P, 1, 0, P, P, 32, 0, None, 0, P, BF, None) == SHAPE
    assert f(P, 1, 124160, P, P, 0, 0, None, 0, P, BF, None) == LIMIT
    assert f(P, 1, 124160, P, P, 1025, 0, None, 0, P, BF, None) == LIMIT
    assert f(P + 2, 1, 124160, P, P, 32, 0, None, 0, P, BF, None) == ALIGN     # y not 16-byte aligned
    assert f(P, 1, 124160, P, P, 32, 0, None, 0, P + 8, F32, None) == ALIGN    # out not 16-byte aligned
    assert f(P, 1, 124160, P, P, 32, 0, ODD, F32, P, BF, None) == ALIGN        # fp32 bias misaligned


def test_fp8_entry_points_reject_before_launch():
    lib = i2h.lib()
    # W8, wscale, ldw, N, K, packed, S, ZS, stream
    assert lib.i2h_pack_fp8(P, None, 5120, 100, 5120, P, P, P, None) == ARG        # no scale
    assert lib.i2h_pack_fp8(P, P, 5120, 100, 5000, P, P, P, None) == SHAPE         # K % 512
    assert lib.i2h_pack_fp8(P + 4, P, 5120, 100, 5120, P, P, P, None) == ALIGN     # W8 not 8-byte aligned
    assert lib.i2h_pack_fp8(P, P + 2, 5120, 100, 5120, P, P, P, None) == ALIGN     # scale misaligned
    # x, M, W8, ldw, N, K, wscale, sel, R, exact, stream
    assert lib.i2h_rerank_fp8(P, 1, P, 5120, 100, 5120, None, P, 32, P, None) == ARG
    assert lib.i2h_rerank_fp8(P, 1, P, 5120, 100, 5120, P, P, 0, P, None) == LIMIT
    assert lib.i2h_rerank_fp8(P, 1, P, 5124, 100, 5120, P, P, 32, P, None) == ALIGN  # ldw % 8
    f = lib.i2h_select_rerank_topk_fp8
    # cand_score, cand_idx, M, nblk, kcand, R, x, W8, wscale, ldw, N, K, k, sel, exact, out_idx, out_val, stream
    assert f(P, P, 1, 1940, 8, 32, P, P, None, 5120, 124160, 5120, 1, None, None, P, P, None) == ARG
    assert f(P, P, 1, 1940, 8, 65, P, P, P, 5120, 124160, 5120, 1, None, None, P, P, None) == LIMIT
    assert f(P, P, 1, 1940, 8, 32, P, P + 4, P, 5120, 124160, 5120, 1, None, None, P, P, None) == ALIGN


def test_int4_entry_points_reject_before_launch():
    lib = i2h.lib()
    # W, ldw, N, K, packed4, S, ZS, stream
    assert lib.i2h_pack4(None, 5120, 100, 5120, P, P, P, None) == ARG
    assert lib.i2h_pack4(P, 5120, 100, 5000, P, P, P, None) == SHAPE        # K % 256
    assert lib.i2h_pack4(P, 5120, 100, 5376, P, P, P, None) == SHAPE        # ldw < K
    assert lib.i2h_pack4(P + 4, 5120, 100, 5120, P, P, P, None) == ALIGN    # W not 8-byte aligned
    # x, xs, M, packed4, S, ZS, N, K, kcand, cand_score, cand_idx, y, stream
    f = lib.i2h_coarse4_topk
    assert f(P, None, 1, P, P, P, 124160, 5120, 1, P, P, None, None) == ARG  # xs required
    assert f(P, P, 1, P, P, P, 124160, 5000, 1, P, P, None, None) == SHAPE
    assert f(P, P, 1, P, P, P, 124160, 5120, 0, P, P, None, None) == LIMIT
    assert f(P, P, 1, P, P, P, 124160, 5120, 65, P, P, None, None) == LIMIT
    assert f(P + 8, P, 1, P, P, P, 124160, 5120, 1, P, P, None, None) == ALIGN


def test_select_tokens_rejects_before_launch():
    f = i2h.lib().i2h_select_tokens
    # y, M, N, R, sel, workspace, workspace_bytes, stream
    assert f(None, 1, 100, 32, P, None, 0, None) == ARG
    assert f(P, 1, 100, 32, None, None, 0, None) == ARG
    assert f(P, 0, 100, 32, P, None, 0, None) == SHAPE
    assert f(P, 65536, 100, 32, P, None, 0, None) == SHAPE
    assert f(P, 1, 0, 32, P, None, 0, None) == SHAPE
    assert f(P, 1, 1 << 31, 32, P, None, 0, None) == SHAPE
    assert f(P, 1, 100, 0, P, None, 0, None) == LIMIT
    assert f(P, 1, 100, 1025, P, None, 0, None) == LIMIT
    assert f(P + 1, 1, 100, 32, P, None, 0, None) == ALIGN
    assert f(P, 1, 100, 32, P + 2, None, 0, None) == ALIGN
    assert f(P, 1, 124160, 32, P, P + 4, 1 << 20, None) == ALIGN
    wsb = i2h.lib().i2h_select_tokens_workspace_bytes
    assert wsb(1, 124160, 32) == 8 * 32 * 8                 # 8 chunks of 16384 entries
    assert wsb(2, 248320, 1024) == 0                         # 16 x 1024 keys exceed one merge
    assert wsb(1, 16384, 32) == 0                            # one chunk: one workgroup
    assert f(P, 1, 124160, 32, P, P, 8 * 32 * 8 - 1, None) == WS


def test_variant_entry_points_reject_before_launch():
    lib = i2h.lib()
    # W, ldw, N, K, group, layout, packed, S, ZS, stream
    f = lib.i2h_pack_variant
    assert f(None, 5120, 10, 5120, 128, 0, P, P, P, None) == ARG
    assert f(P, 5120, 10, 5120, 96, 0, P, P, P, None) == ARG         # group 64 or 128
    assert f(P, 5120, 10, 5120, 128, 2, P, P, P, None) == ARG        # layout 0 or 1
    assert f(P, 5120, 10, 5000, 128, 0, P, P, P, None) == SHAPE      # K % (4 group)
    assert f(P, 5120, 10, 5376, 64, 1, P, P, P, None) == SHAPE       # ldw < K
    assert f(P + 1, 5120, 10, 5120, 64, 1, P, P, P, None) == ALIGN
    # x, M, K, group, xs, stream
    g = lib.i2h_xsum_group
    assert g(P, 1, 5120, 32, P, None) == ARG
    assert g(P, 1, 5100, 64, P, None) == SHAPE
    # x, xs, M, packed, S, ZS, N, K, group, layout, scaling, kcand, cand_score, cand_idx, stream
    c = lib.i2h_coarse_variant_topk
    assert c(None, None, 1, P, P, P, 1000, 5120, 128, 0, 0, 8, P, P, None) == ARG
    assert c(P, P, 17, P, P, P, 1000, 5120, 128, 0, 0, 8, P, P, None) == SHAPE      # M <= 16
    assert c(P, P, 1, P, P, P, 1000, 1024, 128, 0, 0, 8, P, P, None) == SHAPE       # K = 512 or 5120
    assert c(P, P, 1, P, P, P, 1000, 5120, 64, 1, 2, 8, P, P, None) == ARG          # scaling 0 or 1
    # one property changed at a time: group 64 with contiguous-4, or with the weight tile
    assert c(P, P, 1, P, P, P, 1000, 5120, 64, 1, 0, 8, P, P, None) == ARG
    assert c(P, P, 1, P, P, P, 1000, 5120, 64, 0, 1, 8, P, P, None) == ARG
    assert c(P, P, 1, P, P, P, 1000, 5120, 128, 1, 1, 8, P, P, None) == ARG
    assert c(P, P, 1, P, P, P, 1000, 5120, 64, 0, 0, 0, P, P, None) == LIMIT
    assert c(P + 8, P, 1, P, P, P, 1000, 5120, 64, 0, 0, 8, P, P, None) == ALIGN
    assert c(P, P, 1, P, P + 2, P, 1000, 5120, 128, 1, 0, 8, P, P, None) == ALIGN   # S 16-byte aligned


def test_head_noalloc_statuses():
    """i2h_head_noalloc takes i2h_head's checks, then rejects a call too large for its scratch;
    all before any HIP call."""
    h = i2h.lib().i2h_head_noalloc
    SCRATCH = -8
    assert h(P, 200, P, P, P, P, 5120, 248320, 5120, 8, 32, 1, P, P, None, None) == SCRATCH
    assert h(P, 400, P, P, P, P, 5120, 124160, 5120, 8, 32, 1, P, P, None, None) == SCRATCH
    assert h(None, 1, P, P, P, P, 5120, 124160, 5120, 8, 32, 1, P, P, None, None) == ARG
    assert h(P, 1, P, P, P, P, 5120, 124160, 5000, 8, 32, 1, P, P, None, None) == SHAPE
    assert h(P, 1, P, P, P, P, 5120, 124160, 5120, 8, 32, 33, P, P, None, None) == LIMIT
    assert h(ODD, 1, P, P, P, P, 5120, 124160, 5120, 8, 32, 1, P, P, None, None) == ALIGN
    # I2H_NOALLOC_SCRATCH_BYTES, 26 MiB: the full vocabulary fits up to 96 rows, the vocab slice up to 128
    assert i2h.workspace_bytes(96, 248320, 5120, 8, 32) <= 26 << 20 < i2h.workspace_bytes(200, 248320, 5120, 8, 32)
    assert i2h.workspace_bytes(128, 124160, 5120, 8, 32) <= 26 << 20 < i2h.workspace_bytes(400, 124160, 5120, 8, 32)
