"""Python binding of libi2h, the int2 speculative-draft LM head for MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels. PyTorch provides the
device memory and the stream; each call enqueues on torch's current stream of the tensors'
device and returns without synchronising. The names follow the C ABI in include/i2h.h.

    packed, S, ZS = pack(W)                       # W bf16 [N, K] on the GPU
    idx, val = head(x, packed, S, ZS, W, k=1)     # argmax per row of x bf16 [M, K]
    idx, val = head(x, packed, S, ZS, W, k=16)    # top-16 drawn from the reranked tokens
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["I2HError", "lib", "library_path", "sizes", "pack", "xsum", "coarse_topk", "select",
           "rerank", "finalize", "rerank_topk", "select_rerank_topk", "coarse_sums_x", "workspace_bytes", "head",
           "head_noalloc",
           "logits", "pack_fp8", "rerank_fp8", "select_rerank_topk_fp8", "pack4", "coarse4_topk",
           "select_tokens", "pack_variant", "xsum_group", "coarse_variant_topk", "GROUP",
           "BLOCK_N"]

GROUP = 128
BLOCK_N = 64
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libi2h.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_SIGNATURES = {
    "i2h_version": ([], _INT),
    "i2h_strerror": ([_INT], ctypes.c_char_p),
    "i2h_last_hip_error": ([], _INT),
    "i2h_sizes": ([_I64, _I64, _P, _P], _INT),
    "i2h_pack": ([_P, _I64, _I64, _I64, _P, _P, _P, _P], _INT),
    "i2h_xsum": ([_P, _I64, _I64, _P, _P], _INT),
    "i2h_coarse_topk": ([_P, _P, _I64, _P, _P, _P, _I64, _I64, _INT, _P, _P, _P, _P], _INT),
    "i2h_select": ([_P, _P, _I64, _I64, _INT, _INT, _P, _P], _INT),
    "i2h_rerank": ([_P, _I64, _P, _I64, _I64, _I64, _P, _INT, _P, _P], _INT),
    "i2h_finalize": ([_P, _P, _I64, _INT, _INT, _P, _P, _P], _INT),
    "i2h_workspace_bytes": ([_I64, _I64, _I64, _INT, _INT], _I64),
    "i2h_coarse_sums_x": ([_I64, _I64], _INT),
    "i2h_rerank_topk": ([_P, _I64, _P, _I64, _I64, _I64, _P, _INT, _INT, _P, _P, _P, _P], _INT),
    "i2h_select_rerank_topk": ([_P, _P, _I64, _I64, _INT, _INT, _P, _P, _I64, _I64, _I64, _INT, _P, _P, _P, _P,
                                _P], _INT),
    "i2h_head": ([_P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _INT, _INT, _P, _P, _P, _P,
                  _I64, _P], _INT),
    "i2h_head_noalloc": ([_P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _INT, _INT, _P, _P, _P, _P], _INT),
    "i2h_logits": ([_P, _I64, _I64, _P, _P, _INT, _INT, _P, _INT, _P, _INT, _P], _INT),
    "i2h_pack_fp8": ([_P, _P, _I64, _I64, _I64, _P, _P, _P, _P], _INT),
    "i2h_pack4": ([_P, _I64, _I64, _I64, _P, _P, _P, _P], _INT),
    "i2h_coarse4_topk": ([_P, _P, _I64, _P, _P, _P, _I64, _I64, _INT, _P, _P, _P, _P], _INT),
    "i2h_select_tokens": ([_P, _I64, _I64, _INT, _P, _P, _I64, _P], _INT),
    "i2h_select_tokens_workspace_bytes": ([_I64, _I64, _INT], _I64),
    "i2h_pack_variant": ([_P, _I64, _I64, _I64, _INT, _INT, _P, _P, _P, _P], _INT),
    "i2h_xsum_group": ([_P, _I64, _I64, _INT, _P, _P], _INT),
    "i2h_coarse_variant_topk": ([_P, _P, _I64, _P, _P, _P, _I64, _I64, _INT, _INT, _INT, _INT, _P, _P, _P], _INT),
    "i2h_rerank_fp8": ([_P, _I64, _P, _I64, _I64, _I64, _P, _P, _INT, _P, _P], _INT),
    "i2h_select_rerank_topk_fp8": ([_P, _P, _I64, _I64, _INT, _INT, _P, _P, _P, _I64, _I64, _I64, _INT, _P, _P, _P,
                                    _P, _P], _INT),
}
_DTYPE_CODES = {None: 0, torch.bfloat16: 1, torch.float16: 2, torch.float32: 3}


class I2HError(RuntimeError):
    """A libi2h call returned a negative status."""

    def __init__(self, name: str, status: int):
        msg = lib().i2h_strerror(status).decode()
        if status == -6:
            msg += f" (hipError {lib().i2h_last_hip_error()})"
        super().__init__(f"{name}: {msg} [status {status}]")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libi2h. Raises if the library has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"libi2h.so not found at {_LIB_PATH}; build it with "
                              "`python -m bit_quantized_lm_int2_amd.build` (needs hipcc)")
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def _check(name: str, status: int) -> None:
    if status != 0:
        raise I2HError(name, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _rows(t: torch.Tensor, name: str) -> int:
    """Row stride of a 2-D tensor whose rows are contiguous."""
    if t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    return t.stride(0)


def _dense(t: torch.Tensor, name: str) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _head_shapes(x, packed, S, ZS, xs=None):
    """(M, N, K) after checking that the stored head matches x."""
    M, K = x.shape
    N = packed.shape[0]
    _shape(packed, "packed", (N, K // 4))
    _need(S, "S", torch.bfloat16, 2)
    _need(ZS, "ZS", torch.bfloat16, 2)
    _shape(S, "S", (N, K // GROUP))
    _shape(ZS, "ZS", (N, K // GROUP))
    if xs is not None:
        _need(xs, "xs", torch.float32, 2)
        _shape(xs, "xs", (M, K // GROUP))
    return M, N, K


def sizes(N: int, K: int):
    pb, se = ctypes.c_int64(), ctypes.c_int64()
    _check("i2h_sizes", lib().i2h_sizes(N, K, ctypes.byref(pb), ctypes.byref(se)))
    return pb.value, se.value


def pack(W: torch.Tensor, out=None):
    """(packed u8 [N, K/4], S bf16 [N, K/128], ZS bf16 [N, K/128]) for a bf16 head W [N, K]."""
    _need(W, "W", torch.bfloat16, 2)
    N, K = W.shape
    if out is None:
        packed = torch.empty(N, K // 4, dtype=torch.uint8, device=W.device)
        S = torch.empty(N, K // GROUP, dtype=torch.bfloat16, device=W.device)
        ZS = torch.empty_like(S)
    else:
        packed, S, ZS = out
    _shape(packed, "packed", (N, K // 4))
    _shape(S, "S", (N, K // GROUP))
    _shape(ZS, "ZS", (N, K // GROUP))
    for t, nm in ((packed, "packed"), (S, "S"), (ZS, "ZS")):
        _dense(t, nm)
    _check("i2h_pack", lib().i2h_pack(_ptr(W), _rows(W, "W"), N, K, _ptr(packed), _ptr(S), _ptr(ZS),
                                      _stream(W)))
    return packed, S, ZS


def xsum(x: torch.Tensor, out=None) -> torch.Tensor:
    _need(x, "x", torch.bfloat16, 2)
    _dense(x, "x")
    M, K = x.shape
    xs = out if out is not None else torch.empty(M, K // GROUP, dtype=torch.float32, device=x.device)
    _shape(xs, "xs", (M, K // GROUP))
    _check("i2h_xsum", lib().i2h_xsum(_ptr(x), M, K, _ptr(xs), _stream(x)))
    return xs


def coarse_sums_x(M: int, K: int) -> bool:
    """True when coarse_topk may be given xs=None (the kernel sums the groups of x itself)."""
    return bool(lib().i2h_coarse_sums_x(M, K))


def coarse_topk(x, xs, packed, S, ZS, kcand: int = 8, want_y: bool = False):
    """(cand_score fp32 [M, NBLK*kcand], cand_idx int32 [M, NBLK*kcand], y bf16 [M, N] or None).

    xs may be None when coarse_sums_x(M, K)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(packed, "packed", torch.uint8, 2)
    for t, nm in ((x, "x"), (xs, "xs"), (packed, "packed"), (S, "S"), (ZS, "ZS")):
        if t is not None:
            _dense(t, nm)
    M, N, K = _head_shapes(x, packed, S, ZS, xs)
    nblk = (N + BLOCK_N - 1) // BLOCK_N
    cs = torch.empty(M, nblk * kcand, dtype=torch.float32, device=x.device)
    ci = torch.empty(M, nblk * kcand, dtype=torch.int32, device=x.device)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device) if want_y else None
    _check("i2h_coarse_topk", lib().i2h_coarse_topk(_ptr(x), _ptr(xs), M, _ptr(packed), _ptr(S), _ptr(ZS),
                                                    N, K, kcand, _ptr(cs), _ptr(ci), _ptr(y), _stream(x)))
    return cs, ci, y


def select(cand_score, cand_idx, kcand: int, R: int) -> torch.Tensor:
    _need(cand_score, "cand_score", torch.float32, 2)
    _need(cand_idx, "cand_idx", torch.int32, 2)
    _dense(cand_score, "cand_score")
    _dense(cand_idx, "cand_idx")
    M, ncand = cand_score.shape
    _shape(cand_idx, "cand_idx", (M, ncand))
    if ncand % kcand:
        raise ValueError("candidate count is not a multiple of kcand")
    sel = torch.empty(M, R, dtype=torch.int32, device=cand_score.device)
    _check("i2h_select", lib().i2h_select(_ptr(cand_score), _ptr(cand_idx), M, ncand // kcand, kcand, R,
                                          _ptr(sel), _stream(cand_score)))
    return sel


def rerank(x, W, sel) -> torch.Tensor:
    _need(x, "x", torch.bfloat16, 2)
    _need(W, "W", torch.bfloat16, 2)
    _need(sel, "sel", torch.int32, 2)
    _dense(x, "x")
    _dense(sel, "sel")
    M, K = x.shape
    R = sel.shape[1]
    _shape(sel, "sel", (M, R))
    if W.shape[1] != K:
        raise ValueError("W must have K columns")
    ex = torch.empty(M, R, dtype=torch.float32, device=x.device)
    _check("i2h_rerank", lib().i2h_rerank(_ptr(x), M, _ptr(W), _rows(W, "W"), W.shape[0], K, _ptr(sel), R,
                                          _ptr(ex), _stream(x)))
    return ex


def finalize(exact, sel, k: int = 1):
    _need(exact, "exact", torch.float32, 2)
    _need(sel, "sel", torch.int32, 2)
    _dense(exact, "exact")
    _dense(sel, "sel")
    M, R = exact.shape
    _shape(sel, "sel", (M, R))
    oi = torch.empty(M, k, dtype=torch.int32, device=exact.device)
    ov = torch.empty(M, k, dtype=torch.float32, device=exact.device)
    _check("i2h_finalize", lib().i2h_finalize(_ptr(exact), _ptr(sel), M, R, k, _ptr(oi), _ptr(ov),
                                              _stream(exact)))
    return oi, ov


def rerank_topk(x, W, sel, k: int = 1, exact: torch.Tensor | None = None):
    """Rerank then finalize in one call: (idx int32 [M, k], val fp32 [M, k])."""
    _need(x, "x", torch.bfloat16, 2)
    _need(W, "W", torch.bfloat16, 2)
    _need(sel, "sel", torch.int32, 2)
    _dense(x, "x")
    _dense(sel, "sel")
    M, K = x.shape
    R = sel.shape[1]
    _shape(sel, "sel", (M, R))
    if W.shape[1] != K:
        raise ValueError("W must have K columns")
    if exact is None and R > 64:
        exact = torch.empty(M, R, dtype=torch.float32, device=x.device)
    if exact is not None:
        _need(exact, "exact", torch.float32, 2)
        _shape(exact, "exact", (M, R))
    oi = torch.empty(M, k, dtype=torch.int32, device=x.device)
    ov = torch.empty(M, k, dtype=torch.float32, device=x.device)
    _check("i2h_rerank_topk", lib().i2h_rerank_topk(_ptr(x), M, _ptr(W), _rows(W, "W"), W.shape[0], K, _ptr(sel),
                                                    R, k, _ptr(exact), _ptr(oi), _ptr(ov), _stream(x)))
    return oi, ov


def select_rerank_topk(cand_score, cand_idx, kcand: int, R: int, x, W, k: int = 1, want_sel: bool = False):
    """Selection, exact rerank and top-k in one call: (idx int32 [M, k], val fp32 [M, k]) and, with
    want_sel, also (sel int32 [M, R], exact fp32 [M, R])."""
    _need(cand_score, "cand_score", torch.float32, 2)
    _need(cand_idx, "cand_idx", torch.int32, 2)
    _need(x, "x", torch.bfloat16, 2)
    _need(W, "W", torch.bfloat16, 2)
    for t, n in ((cand_score, "cand_score"), (cand_idx, "cand_idx"), (x, "x")):
        _dense(t, n)
    M, ncand = cand_score.shape
    _shape(cand_idx, "cand_idx", (M, ncand))
    _shape(x, "x", (M, x.shape[1]))
    K = x.shape[1]
    if ncand % kcand:
        raise ValueError("candidate count is not a multiple of kcand")
    if W.shape[1] != K:
        raise ValueError("W must have K columns")
    dev = x.device
    oi = torch.empty(M, k, dtype=torch.int32, device=dev)
    ov = torch.empty(M, k, dtype=torch.float32, device=dev)
    sel = torch.empty(M, R, dtype=torch.int32, device=dev) if want_sel else None
    ex = torch.empty(M, R, dtype=torch.float32, device=dev) if want_sel else None
    _check("i2h_select_rerank_topk",
           lib().i2h_select_rerank_topk(_ptr(cand_score), _ptr(cand_idx), M, ncand // kcand, kcand, R, _ptr(x), _ptr(W),
                                        _rows(W, "W"), W.shape[0], K, k, _ptr(sel), _ptr(ex), _ptr(oi), _ptr(ov),
                                        _stream(x)))
    return (oi, ov, sel, ex) if want_sel else (oi, ov)


def workspace_bytes(M: int, N: int, K: int, kcand: int = 8, R: int = 32) -> int:
    n = lib().i2h_workspace_bytes(M, N, K, kcand, R)
    if n < 0:
        raise I2HError("i2h_workspace_bytes", int(n))
    return int(n)


def head(x, packed, S, ZS, W, kcand: int = 8, R: int = 32, k: int = 1, want_y: bool = False,
         workspace: torch.Tensor | None = None, out=None):
    """(idx int32 [M, k], val fp32 [M, k][, y bf16 [M, N]]) for one call of the head."""
    _need(x, "x", torch.bfloat16, 2)
    _need(W, "W", torch.bfloat16, 2)
    _need(packed, "packed", torch.uint8, 2)
    for t, nm in ((x, "x"), (packed, "packed"), (S, "S"), (ZS, "ZS")):
        _dense(t, nm)
    M, N, K = _head_shapes(x, packed, S, ZS)
    if tuple(W.shape) != (N, K):
        raise ValueError(f"W must have shape {(N, K)}, got {tuple(W.shape)}")
    need = workspace_bytes(M, N, K, kcand, R)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    elif workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if out is None:
        oi = torch.empty(M, k, dtype=torch.int32, device=x.device)
        ov = torch.empty(M, k, dtype=torch.float32, device=x.device)
    else:
        oi, ov = out
    y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device) if want_y else None
    _check("i2h_head", lib().i2h_head(_ptr(x), M, _ptr(packed), _ptr(S), _ptr(ZS), _ptr(W), _rows(W, "W"), N, K,
                                      kcand, R, k, _ptr(oi), _ptr(ov), _ptr(y), _ptr(workspace),
                                      workspace.numel(), _stream(x)))
    return (oi, ov, y) if want_y else (oi, ov)


def head_noalloc(x, packed, S, ZS, W, kcand: int = 8, R: int = 32, k: int = 1, out=None, y=None):
    """head() through i2h_head_noalloc: the library's own device scratch instead of a workspace.
    With out = (idx int32 [M, k], val fp32 [M, k]) given (and y, bf16 [M, N], if wanted) this
    allocates nothing."""
    _need(x, "x", torch.bfloat16, 2)
    _need(W, "W", torch.bfloat16, 2)
    _need(packed, "packed", torch.uint8, 2)
    for t, nm in ((x, "x"), (packed, "packed"), (S, "S"), (ZS, "ZS")):
        _dense(t, nm)
    M, N, K = _head_shapes(x, packed, S, ZS)
    if tuple(W.shape) != (N, K):
        raise ValueError(f"W must have shape {(N, K)}, got {tuple(W.shape)}")
    if out is None:
        oi = torch.empty(M, k, dtype=torch.int32, device=x.device)
        ov = torch.empty(M, k, dtype=torch.float32, device=x.device)
    else:
        oi, ov = out
        _need(oi, "idx", torch.int32, 2)
        _need(ov, "val", torch.float32, 2)
        _shape(oi, "idx", (M, k))
        _shape(ov, "val", (M, k))
        _dense(oi, "idx")
        _dense(ov, "val")
    if y is not None:
        _need(y, "y", torch.bfloat16, 2)
        _shape(y, "y", (M, N))
        _dense(y, "y")
    _check("i2h_head_noalloc", lib().i2h_head_noalloc(_ptr(x), M, _ptr(packed), _ptr(S), _ptr(ZS), _ptr(W),
                                                      _rows(W, "W"), N, K, kcand, R, k, _ptr(oi), _ptr(ov),
                                                      _ptr(y), _stream(x)))
    return oi, ov


def logits(y, sel, exact, topk_only: bool = False, bias: torch.Tensor | None = None,
           out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """The drop-in logits row [M, N] of out_dtype: the coarse bf16 row y (or -inf everywhere when
    topk_only; y may then be None), the exact scores written back at the sel tokens, plus the
    embedding bias (bf16, fp16 or fp32 [N]) and the cast to out_dtype. out may be y itself
    (bf16)."""
    _need(sel, "sel", torch.int32, 2)
    _need(exact, "exact", torch.float32, 2)
    M, R = sel.shape
    _shape(exact, "exact", (M, R))
    _dense(sel, "sel")
    _dense(exact, "exact")
    if y is not None:
        _need(y, "y", torch.bfloat16, 2)
        _dense(y, "y")
        if y.shape[0] != M:
            raise ValueError("y and sel must have the same rows")
        N = y.shape[1]
    elif not topk_only:
        raise ValueError("y is needed unless topk_only")
    elif bias is not None:
        N = bias.shape[0]
    elif out is not None:
        N = out.shape[1]
    else:
        raise ValueError("with y None, give bias or out so that N is known")
    if out_dtype not in (torch.bfloat16, torch.float16, torch.float32):
        raise ValueError("out_dtype must be bfloat16, float16 or float32")
    if bias is not None:
        if bias.dtype not in (torch.bfloat16, torch.float16, torch.float32) or tuple(bias.shape) != (N,):
            raise ValueError(f"bias must be a [{N}] bfloat16, float16 or float32 tensor")
        _dense(bias, "bias")
    dev = sel.device
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=dev)
    elif out.dtype != out_dtype or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{M}, {N}] {out_dtype} tensor")
    _check("i2h_logits", lib().i2h_logits(_ptr(y), M, N, _ptr(sel), _ptr(exact), R, int(bool(topk_only)),
                                          _ptr(bias), _DTYPE_CODES[None if bias is None else bias.dtype], _ptr(out),
                                          _DTYPE_CODES[out_dtype], _stream(sel)))
    return out


def _fp8_head(W8, wscale):
    _need(W8, "W8", torch.uint8, 2)
    _need(wscale, "wscale", torch.float32, 1)
    _dense(wscale, "wscale")
    if wscale.shape[0] != W8.shape[0]:
        raise ValueError("wscale must have one entry per row of W8")
    if W8.stride(1) != 1:
        raise ValueError("W8 rows must be contiguous")


def pack_fp8(W8: torch.Tensor, wscale: torch.Tensor, out=None):
    """pack() for an FP8 head: W8 uint8 e4m3 codes [N, K] with a per-row fp32 scale [N]."""
    _fp8_head(W8, wscale)
    N, K = W8.shape
    if out is None:
        packed = torch.empty(N, K // 4, dtype=torch.uint8, device=W8.device)
        S = torch.empty(N, K // GROUP, dtype=torch.bfloat16, device=W8.device)
        ZS = torch.empty_like(S)
    else:
        packed, S, ZS = out
    _shape(packed, "packed", (N, K // 4))
    _shape(S, "S", (N, K // GROUP))
    _shape(ZS, "ZS", (N, K // GROUP))
    for t, nm in ((packed, "packed"), (S, "S"), (ZS, "ZS")):
        _dense(t, nm)
    _check("i2h_pack_fp8", lib().i2h_pack_fp8(_ptr(W8), _ptr(wscale), W8.stride(0), N, K, _ptr(packed), _ptr(S),
                                              _ptr(ZS), _stream(W8)))
    return packed, S, ZS


def rerank_fp8(x, W8, wscale, sel) -> torch.Tensor:
    """rerank() against an FP8 head (W8 uint8 [N, K], wscale fp32 [N])."""
    _need(x, "x", torch.bfloat16, 2)
    _need(sel, "sel", torch.int32, 2)
    _fp8_head(W8, wscale)
    _dense(x, "x")
    _dense(sel, "sel")
    M, K = x.shape
    R = sel.shape[1]
    _shape(sel, "sel", (M, R))
    if W8.shape[1] != K:
        raise ValueError("W8 must have K columns")
    ex = torch.empty(M, R, dtype=torch.float32, device=x.device)
    _check("i2h_rerank_fp8", lib().i2h_rerank_fp8(_ptr(x), M, _ptr(W8), W8.stride(0), W8.shape[0], K, _ptr(wscale),
                                                  _ptr(sel), R, _ptr(ex), _stream(x)))
    return ex


def select_rerank_topk_fp8(cand_score, cand_idx, kcand: int, R: int, x, W8, wscale, k: int = 1,
                           want_sel: bool = False):
    """select_rerank_topk() with the exact scores against an FP8 head."""
    _need(cand_score, "cand_score", torch.float32, 2)
    _need(cand_idx, "cand_idx", torch.int32, 2)
    _need(x, "x", torch.bfloat16, 2)
    _fp8_head(W8, wscale)
    for t, n in ((cand_score, "cand_score"), (cand_idx, "cand_idx"), (x, "x")):
        _dense(t, n)
    M, ncand = cand_score.shape
    _shape(cand_idx, "cand_idx", (M, ncand))
    K = x.shape[1]
    if ncand % kcand:
        raise ValueError("candidate count is not a multiple of kcand")
    if W8.shape[1] != K:
        raise ValueError("W8 must have K columns")
    dev = x.device
    oi = torch.empty(M, k, dtype=torch.int32, device=dev)
    ov = torch.empty(M, k, dtype=torch.float32, device=dev)
    sel = torch.empty(M, R, dtype=torch.int32, device=dev) if want_sel else None
    ex = torch.empty(M, R, dtype=torch.float32, device=dev) if want_sel else None
    _check("i2h_select_rerank_topk_fp8",
           lib().i2h_select_rerank_topk_fp8(_ptr(cand_score), _ptr(cand_idx), M, ncand // kcand, kcand, R, _ptr(x),
                                            _ptr(W8), _ptr(wscale), W8.stride(0), W8.shape[0], K, k, _ptr(sel),
                                            _ptr(ex), _ptr(oi), _ptr(ov), _stream(x)))
    return (oi, ov, sel, ex) if want_sel else (oi, ov)


def pack4(W: torch.Tensor, out=None):
    """The int4 head of a bf16 head W [N, K]: (packed4 u8 [N, K/2], S bf16 [N, K/128], ZS)."""
    _need(W, "W", torch.bfloat16, 2)
    N, K = W.shape
    if out is None:
        packed = torch.empty(N, K // 2, dtype=torch.uint8, device=W.device)
        S = torch.empty(N, K // GROUP, dtype=torch.bfloat16, device=W.device)
        ZS = torch.empty_like(S)
    else:
        packed, S, ZS = out
    _shape(packed, "packed4", (N, K // 2))
    _shape(S, "S", (N, K // GROUP))
    _shape(ZS, "ZS", (N, K // GROUP))
    for t, nm in ((packed, "packed4"), (S, "S"), (ZS, "ZS")):
        _dense(t, nm)
    _check("i2h_pack4", lib().i2h_pack4(_ptr(W), _rows(W, "W"), N, K, _ptr(packed), _ptr(S), _ptr(ZS), _stream(W)))
    return packed, S, ZS


def coarse4_topk(x, xs, packed4, S, ZS, kcand: int = 1, want_y: bool = False):
    """(cand_score fp32 [M, NBLK*kcand], cand_idx int32 [M, NBLK*kcand][, y bf16 [M, N]]) of the
    int4 head; xs from xsum(x)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(packed4, "packed4", torch.uint8, 2)
    _need(xs, "xs", torch.float32, 2)
    for t, nm in ((x, "x"), (xs, "xs"), (packed4, "packed4"), (S, "S"), (ZS, "ZS")):
        _dense(t, nm)
    M, K = x.shape
    N = packed4.shape[0]
    _shape(packed4, "packed4", (N, K // 2))
    _shape(S, "S", (N, K // GROUP))
    _shape(ZS, "ZS", (N, K // GROUP))
    _shape(xs, "xs", (M, K // GROUP))
    nblk = (N + BLOCK_N - 1) // BLOCK_N
    cs = torch.empty(M, nblk * kcand, dtype=torch.float32, device=x.device)
    ci = torch.empty(M, nblk * kcand, dtype=torch.int32, device=x.device)
    y = torch.empty(M, N, dtype=torch.bfloat16, device=x.device) if want_y else None
    _check("i2h_coarse4_topk", lib().i2h_coarse4_topk(_ptr(x), _ptr(xs), M, _ptr(packed4), _ptr(S), _ptr(ZS), N, K,
                                                      kcand, _ptr(cs), _ptr(ci), _ptr(y), _stream(x)))
    return (cs, ci, y) if want_y else (cs, ci)


def select_tokens(y, R: int, chunked: bool = True):
    """sel int32 [M, R]: the R largest entries of each bf16 row of y (value descending, lower
    index first on ties), -1 past a row's end. chunked=False takes one workgroup per row."""
    _need(y, "y", torch.bfloat16, 2)
    _dense(y, "y")
    M, N = y.shape
    sel = torch.empty(M, R, dtype=torch.int32, device=y.device)
    nws = lib().i2h_select_tokens_workspace_bytes(M, N, R) if chunked else 0
    if nws < 0:
        raise I2HError("i2h_select_tokens_workspace_bytes", nws)
    ws = torch.empty(nws, dtype=torch.uint8, device=y.device) if nws > 0 else None
    _check("i2h_select_tokens", lib().i2h_select_tokens(_ptr(y), M, N, R, _ptr(sel), _ptr(ws), nws, _stream(y)))
    return sel


_LAYOUTS = {"quarter": 0, "contiguous": 1}
_SCALINGS = {"accumulator": 0, "tile": 1}


def pack_variant(W, group: int = GROUP, layout: str = "quarter"):
    """(packed uint8 [N, K/4], S bf16 [N, K/group], ZS bf16 [N, K/group]) at group 64 or 128 in
    the quarter-split or contiguous-4 layout."""
    _need(W, "W", torch.bfloat16, 2)
    N, K = W.shape
    ldw = _rows(W, "W")
    packed = torch.empty(N, K // 4, dtype=torch.uint8, device=W.device)
    S = torch.empty(N, K // group, dtype=torch.bfloat16, device=W.device)
    ZS = torch.empty(N, K // group, dtype=torch.bfloat16, device=W.device)
    _check("i2h_pack_variant", lib().i2h_pack_variant(_ptr(W), ldw, N, K, group, _LAYOUTS[layout], _ptr(packed),
                                                      _ptr(S), _ptr(ZS), _stream(W)))
    return packed, S, ZS


def xsum_group(x, group: int = GROUP):
    """xs fp32 [M, K/group]: the sums of x over each group of `group` k."""
    _need(x, "x", torch.bfloat16, 2)
    _dense(x, "x")
    M, K = x.shape
    xs = torch.empty(M, K // group, dtype=torch.float32, device=x.device)
    _check("i2h_xsum_group", lib().i2h_xsum_group(_ptr(x), M, K, group, _ptr(xs), _stream(x)))
    return xs


def coarse_variant_topk(x, xs, packed, S, ZS, group: int = GROUP, layout: str = "quarter",
                        scaling: str = "accumulator", kcand: int = 8):
    """(cand_score fp32 [M, NBLK*kcand], cand_idx int32 [M, NBLK*kcand]) of a variant head."""
    _need(x, "x", torch.bfloat16, 2)
    _need(packed, "packed", torch.uint8, 2)
    for t, nm in ((x, "x"), (packed, "packed"), (S, "S"), (ZS, "ZS")):
        _dense(t, nm)
    M, K = x.shape
    N = packed.shape[0]
    _shape(packed, "packed", (N, K // 4))
    _shape(S, "S", (N, K // group))
    _shape(ZS, "ZS", (N, K // group))
    if xs is not None:
        _need(xs, "xs", torch.float32, 2)
        _dense(xs, "xs")
        _shape(xs, "xs", (M, K // group))
    nblk = (N + BLOCK_N - 1) // BLOCK_N
    cs = torch.empty(M, nblk * kcand, dtype=torch.float32, device=x.device)
    ci = torch.empty(M, nblk * kcand, dtype=torch.int32, device=x.device)
    _check("i2h_coarse_variant_topk",
           lib().i2h_coarse_variant_topk(_ptr(x), _ptr(xs), M, _ptr(packed), _ptr(S), _ptr(ZS), N, K, group,
                                         _LAYOUTS[layout], _SCALINGS[scaling], kcand, _ptr(cs), _ptr(ci),
                                         _stream(x)))
    return cs, ci
