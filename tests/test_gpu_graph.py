"""The whole paths captured into a HIP graph.

The library only enqueues kernels on the caller's stream (no allocation, no
synchronization, no memset), so its calls can be captured into a graph.  Each
whole path is captured once, the graph is replayed several times with the
program's own eager work and synchronizations in between, and every replay must
give the bytes of the eager call.  Covered: the short single-launch path, the
two-kernel int8 path with rotation, the gate/up SwiGLU, fp8, and the gate/up
SwiGLU quantized for the next linear (three kernels).
"""
import pytest
import torch

import workloads as W
from parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    import w8a8_quantized_linear_amd as lib
    return lib


def _case(lib, kind, M, K, N, rot, seed):
    wl = W.custom(kind, M, K, N, rot, bias=kind != "fp8", seed=seed)
    inp = W.make_inputs(wl)
    dev = torch.device("cuda")
    quant = lib.w8a8_quantize_act_fp8 if kind == "fp8" else lib.w8a8_quantize_act
    wq, s_ch = quant(inp.w.to(dev), rot)
    wp = lib.w8a8_pack_weight(wq)
    bias = None if inp.bias is None else inp.bias.to(dev)
    return wl, inp.x.to(dev), wp, s_ch, bias


CASES = [
    ("linear", 298, 1024, 1024, 0, "short single launch"),
    ("linear", 1502, 1024, 512, 128, "quantizer + GEMM, rotated"),
    ("gateup", 300, 512, 384, 0, "gate/up SwiGLU"),
    ("fp8", 260, 512, 256, 0, "fp8"),
    ("quant", 300, 512, 384, 0, "gate/up SwiGLU quantized for the next linear"),
]


@pytest.mark.parametrize("kind,M,K,N,rot,what", CASES, ids=[c[5] for c in CASES])
def test_capture_and_replay(lib, kind, M, K, N, rot, what):
    say(f"graph: {what} M={M} K={K} N={N} rot={rot}")
    dev = torch.device("cuda")
    wl, x, wp, s_ch, bias = _case(lib, "gateup" if kind == "quant" else kind, M, K, N, rot, seed=M + N)
    if kind == "quant":
        ws = torch.empty(lib.swiglu_quant_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
        q_out = torch.zeros(lib.packed_bytes(M, N), dtype=torch.int8, device=dev)
        s_out = torch.zeros(M, dtype=torch.float32, device=dev)

        def call():
            lib.w8a8_gateup_swiglu_quant_packed(x, wp, N, s_ch, bias, rot_in=rot, rot_out=128, workspace=ws,
                                                q_out=q_out, s_out=s_out)

        outs = (q_out, s_out)
    else:
        fn = {"linear": lib.w8a8_linear_packed, "gateup": lib.w8a8_gateup_swiglu_packed,
              "fp8": lib.w8a8_fp8_linear_packed}[kind]
        ws = torch.empty(lib.workspace_bytes(M, K), dtype=torch.uint8, device=dev)
        y = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)

        def call():
            fn(x, wp, N, s_ch, bias, rot_block=rot, workspace=ws, out=y)

        outs = (y,)
    call()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for o in outs:
            o.zero_()
        with torch.cuda.graph(g, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.zero_()                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs from the eager call"
    say(f"  4 replays identical to the eager call")
