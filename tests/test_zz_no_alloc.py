"""i2h_head_noalloc (the library's static device scratch in place of a caller workspace) against
i2h_head, through the C ABI: bit-identical outputs on calls in a row, each smaller than the one
before, so every call after the first meets the scratch as the previous call left it."""
import numpy as np
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def i2h():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_quantized_lm_int2_amd as lib
    lib.lib()
    return lib


def _case(i2h, M, N, K, k, seed):
    x = si.gen_x(M, K, outliers=8, seed=seed).to(DEV)
    W = si.gen_weight(N, K, seed=seed + 1).to(DEV)
    p, S, ZS = i2h.pack(W)
    return x, W, p, S, ZS


def test_head_noalloc_matches_head(i2h):
    # largest first: the 64-row tile over a vocab slice (7.9 MB of candidates in the scratch),
    # then the split tail at one row (its arrival counters land where the first call wrote
    # candidates), then 16 rows at another K and N
    for M, N, K, k in ((64, 124160, 5120, 16), (1, 4133, 5120, 1), (16, 20011, 512, 4)):
        print(f"noalloc M={M} N={N} K={K} k={k}", flush=True)
        x, W, p, S, ZS = _case(i2h, M, N, K, k, seed=M + N)
        want_i, want_v = i2h.head(x, p, S, ZS, W, k=k)
        oi = torch.full((M, k), -7, dtype=torch.int32, device=DEV)
        ov = torch.zeros(M, k, dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()
        allocs = torch.cuda.memory_stats()["allocation.all.allocated"]  # requests made so far
        got_i, got_v = i2h.head_noalloc(x, p, S, ZS, W, k=k, out=(oi, ov))
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats()["allocation.all.allocated"] == allocs
        assert got_i.data_ptr() == oi.data_ptr()
        assert torch.equal(got_i, want_i) and torch.equal(got_v, want_v), f"M={M} N={N} K={K}"
        assert int((got_i >= 0).sum()) == M * k


def test_head_noalloc_twice_with_y(i2h):
    """Two calls in a row on one input, the second with the coarse row requested: both equal
    i2h_head's outputs, and y equals i2h_head's y."""
    M, N, K = 5, 9000, 5120
    x, W, p, S, ZS = _case(i2h, M, N, K, 16, seed=77)
    want_i, want_v, want_y = i2h.head(x, p, S, ZS, W, k=16, want_y=True)
    for call in range(2):
        y = torch.zeros(M, N, dtype=torch.bfloat16, device=DEV) if call else None
        got_i, got_v = i2h.head_noalloc(x, p, S, ZS, W, k=16, y=y)
        torch.cuda.synchronize()
        assert torch.equal(got_i, want_i) and torch.equal(got_v, want_v), f"call {call}"
        if y is not None:
            assert torch.equal(y, want_y)


def test_head_noalloc_rejects_oversized_call(i2h):
    x = torch.zeros(200, 512, dtype=torch.bfloat16, device=DEV)
    W = torch.zeros(248320, 512, dtype=torch.bfloat16, device=DEV)
    p = torch.zeros(248320, 128, dtype=torch.uint8, device=DEV)
    S = torch.zeros(248320, 4, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(i2h.I2HError) as e:
        i2h.head_noalloc(x, p, S, S, W)
    assert e.value.status == -8
