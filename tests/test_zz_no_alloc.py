"""The int8 whole path without a workspace (w8a8_linear_packed_noalloc): its outputs
equal w8a8_linear_packed's byte for byte, on two calls in a row into the library's
fixed scratch array, the second with a smaller input; a call beyond the array's
size is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import bf16_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd as lib
    return lib


def _case(lib, M, K, N, rot, seed):
    wl = W.custom("linear", M, K, N, rot, bias=True, seed=seed)
    inp = W.make_inputs(wl)
    dev = torch.device("cuda")
    wq, s_ch = lib.w8a8_quantize_act(inp.w.to(dev), rot)
    return inp.x.to(dev), lib.w8a8_pack_weight(wq), s_ch, inp.bias.to(dev)


def test_noalloc_matches_the_workspace_entry_point(lib):
    # first call: 1,502 x 4,096 x 4,096 rotated (two kernels, 6.2 MB of scratch);
    # second: 298 x 1,024 x 1,024 (the single-launch short path), smaller, same array
    for M, K, N, rot in ((1502, 4096, 4096, 128), (298, 1024, 1024, 0), (700, 2048, 520, 128)):
        say(f"noalloc M={M} K={K} N={N} rot={rot}")
        x, wp, s_ch, bias = _case(lib, M, K, N, rot, seed=M + K)
        y_na = lib.w8a8_linear_packed_noalloc(x, wp, N, s_ch, bias, rot_block=rot)
        ws = torch.empty(lib.workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
        y_ws = lib.w8a8_linear_packed(x, wp, N, s_ch, bias, rot_block=rot, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y_na), bf16_bits(y_ws)), f"M={M}: outputs differ"
        # and again after the other call has used the array (its last contents are stale)
        y2 = lib.w8a8_linear_packed_noalloc(x, wp, N, s_ch, bias, rot_block=rot)
        torch.cuda.synchronize()
        assert torch.equal(y2, y_ws)


def test_noalloc_refuses_more_than_the_array(lib):
    from w8a8_quantized_linear_amd import W8A8Error
    M, K, N = 4096, 16384, 8
    assert lib.workspace_bytes(M, K) > lib.NOALLOC_MAX_WORKSPACE
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    wp = torch.zeros(lib.packed_bytes(N, K), dtype=torch.int8, device="cuda")
    s_ch = torch.ones(N, dtype=torch.float32, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(W8A8Error, match="SCRATCH_TOO_SMALL"):
        lib.w8a8_linear_packed_noalloc(x, wp, N, s_ch, None, out=y)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "nothing is written on an error"
