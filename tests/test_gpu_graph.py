"""GPU test: the calls that allocate nothing can be captured into a HIP graph
and replayed.

torch.cuda.CUDAGraph (HIP graphs on ROCm) captures one call of the library
on the capture stream: the fused forward, the slice forward, the fused
backward and the allocation-free forward on the line kernels.  None of them
allocates or clears memory with a memset, so the graph holds kernel nodes
only.  The graph is replayed three times; before each replay the program
does eager work of its own (a reduction) and overwrites the outputs with 7,
and after it every output must equal the eager call's, bit for bit (the same
kernels on the same inputs).
"""
import pytest

from parity import say
from linear_spatial_propagation_amd import _lib

pytestmark = pytest.mark.gpu

CASES = [
    # (kind, B, C, H, W, groups, cpw, dtype)
    ("fwd", 2, 16, 64, 64, 1, 8, "bf16"),         # fused kernel
    ("fwd", 1, 8, 128, 128, 8, 1, "bf16"),        # slice kernel
    ("bwd", 1, 8, 32, 40, 1, 4, "f32"),           # fused backward
    ("noalloc", 1, 4, 256, 256, 1, 1, "bf16"),    # line kernels on the static scratch
]


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_capture_and_replay(case):
    import torch
    import linear_spatial_propagation_amd as gspn
    kind, B, C, H, W, g, cpw, dtype = case
    say(f"graph case {case}")
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device=dev)
    gen.manual_seed(B * 1000 + C * 10 + H)
    x = torch.randn((B, C, H, W), generator=gen, device=dev).to(dt)
    w = torch.randn((4, B, C // cpw, 3, H, W), generator=gen, device=dev).to(dt)
    lam = torch.rand((B, C, H, W), generator=gen, device=dev).to(dt)
    u = torch.rand((B, C, H, W), generator=gen, device=dev).to(dt)
    gy = torch.randn((B, C, H, W), generator=gen, device=dev).to(dt)
    if kind == "bwd":
        outs = [torch.empty_like(x), torch.empty_like(w), torch.empty_like(x), torch.empty_like(x)]
    else:
        outs = [torch.empty_like(x)]

    def call():
        if kind == "fwd":
            gspn.scan_fwd(x, w, lam, u, groups=g, ch_per_weight=cpw, out=outs[0])
        elif kind == "bwd":
            gspn.scan_bwd(x, w, lam, u, gy, groups=g, ch_per_weight=cpw, out=tuple(outs))
        else:
            rc = _lib.scan_fwd_noalloc_ptr(x.data_ptr(), w.data_ptr(), lam.data_ptr(), u.data_ptr(),
                                           outs[0].data_ptr(), B, C, H, W, groups=g, ch_per_weight=cpw,
                                           dtype=_lib.GSPN_BF16 if dtype == "bf16" else _lib.GSPN_F32,
                                           stream=torch.cuda.current_stream().cuda_stream)
            assert rc == 0, _lib.load().gspn_last_error()

    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs:
            t.fill_(7.0)
        float(torch.randn(1 << 20, device=dev).sum())   # eager work of the program's own, then a sync
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(_bits(t), _bits(r)), f"replay {rep} differs from the eager call"
    say(f"graph case {case}: 3 replays equal the eager call")
