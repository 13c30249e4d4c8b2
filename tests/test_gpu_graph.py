"""The layer calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed: cr_linear_nvfp4,
and the W4A8 / W4A4 (nibble and E2M3 form) layer calls.

cr_linear_nvfp4 allocates nothing and issues no memset; its launches (and, with a second
stream and several weight chunks, its cross-stream events) are recorded into the graph.
Each case replays the graph several times with eager work (fills of the output and the
workspace) and synchronizations in between, and checks every replay against the eager
result, bit for bit."""
import pytest
import torch

import rotated_bit_linear_amd as rbl
import synth
from helpers import dev, say

pytestmark = pytest.mark.gpu

# short batch (decode inside the GEMM, main stream only), one staged chunk, and a chunked
# weight on two streams with events and staged serially
CASES = [(16, 300, 1000, 0, False), (300, 520, 768, 0, True), (300, 1000, 1000, 256 * 1024, True),
         (300, 1000, 1000, 256 * 1024, False)]


@pytest.mark.parametrize("M,N,K,mt,use_aux", CASES, ids=[f"M{c[0]}-N{c[1]}-K{c[2]}-mt{c[3]}-aux{int(c[4])}"
                                                         for c in CASES])
def test_layer_graph_replay(M, N, K, mt, use_aux):
    w = synth.Workload("g", M, N, K, synth.DT_BF16, (synth.DT_BF16,), 41, outlier_frac=0.01)
    x = synth.make_activation(w).to(dev())
    p = synth.make_weight_nvfp4(w)
    cd, sd = p.codes.to(dev()), p.sf.to(dev())
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev())
    ws = torch.empty(rbl.cr_linear_nvfp4_workspace_bytes(M, N, K, mt), dtype=torch.uint8, device=dev())
    out = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    aux = torch.cuda.Stream() if use_aux else None
    say(f"eager cr_linear_nvfp4 M={M} N={N} K={K} max_tile={mt} aux={use_aux}")
    rbl.cr_linear_nvfp4(x, K, False, cd, sd, gs, out, ws, mt, aux_stream=aux)
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # one untimed call on the capture's stream first
        rbl.cr_linear_nvfp4(x, K, False, cd, sd, gs, out, ws, mt, aux_stream=aux)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say(f"capture cr_linear_nvfp4 M={M} N={N} K={K} max_tile={mt} aux={use_aux}")
    with torch.cuda.graph(g):
        rbl.cr_linear_nvfp4(x, K, False, cd, sd, gs, out, ws, mt, aux_stream=aux)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(7.0)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        say(f"replay {i}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager call"


W4_LAYERS = ["w4a8", "w4a4", "w4a4_e2m3"]


@pytest.mark.parametrize("kind", W4_LAYERS)
def test_w4_layer_graph_replay(kind):
    """The W4A8 and W4A4 layer calls (activation preparation into the workspace, then the
    GEMM; no allocation, no memset) captured and replayed like cr_linear_nvfp4."""
    M, N, K = 300, 520, 1000
    w = synth.Workload("g4", M, N, K, synth.DT_BF16, (synth.DT_BF16,), 43, outlier_frac=0.01)
    x = synth.make_activation(w).to(dev())
    wf = synth.make_weight_f32(w).to(dev())
    BT = rbl.CR_FLAG_BLOCK_TRANSPOSED
    if kind == "w4a4_e2m3":
        p, s = rbl.quant_weight_w4_e2m3(wf, K, flags=BT)
        ws = torch.empty(rbl.cr_linear_w4a4_e2m3_workspace_bytes(M, K), dtype=torch.uint8, device=dev())
        call = lambda o: rbl.cr_linear_w4a4_e2m3(x, K, False, p, s, o, ws, flags=BT)  # noqa: E731
    else:
        p, s = rbl.quant_weight_w4(wf, K, flags=BT)
        nbytes = (rbl.cr_linear_w4a8_workspace_bytes if kind == "w4a8" else rbl.cr_linear_w4a4_workspace_bytes)(M, K)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev())
        fn = rbl.cr_linear_w4a8 if kind == "w4a8" else rbl.cr_linear_w4a4
        call = lambda o: fn(x, K, False, p, s, o, ws, flags=BT)  # noqa: E731
    out = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    say(f"eager {kind} M={M} N={N} K={K}")
    call(out)
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say(f"capture {kind} M={M} N={N} K={K}")
    with torch.cuda.graph(g):
        call(out)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(7.0)
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        say(f"replay {i}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{kind}: replay {i} differs from the eager call"
