"""cr_linear_nvfp4_noalloc (the layer on the library's own device scratch, for callers that
cannot allocate) against cr_linear_nvfp4 / cr_linear_nvfp4_ex, through the C ABI.

Three calls in a row, each smaller than the one before, so the second and third run on a
scratch array that still holds the previous call's bytes: a QKV-shaped layer at M = 4096
(the tile bound chosen to fit the scratch, several weight chunks), a SwiGLU layer with a
channel pre-scale and a bias (a small explicit tile bound: two chunks), and a short batch
(decode inside the GEMM).  Every output is bit-identical to the allocating entry point's,
and columns past N are untouched.  Layers whose workspace exceeds the scratch are refused
with CR_ERR_TOO_LARGE before anything is enqueued.
"""
import pytest
import torch

import rotated_bit_linear_amd as rbl
import synth
from helpers import dev, say

pytestmark = pytest.mark.gpu

# name, M, N, K (F for SwiGLU), input dtype, output dtype, swiglu, max_tile_bytes, pre-scale + bias
CALLS = [
    ("qkv-shaped", 4096, 21504, 5376, synth.DT_BF16, synth.DT_BF16, False, 0, False),
    ("swiglu", 300, 1000, 3000, synth.DT_BF16, synth.DT_FP32, True, 256 * 1024, True),
    ("short batch", 40, 500, 1000, synth.DT_FP16, synth.DT_FP16, False, 0, False),
]


def _inputs(M, N, K, x_dt, swiglu, seed):
    w = synth.Workload("noalloc", M, N, K, x_dt, (x_dt,), seed, swiglu=swiglu, outlier_frac=0.01)
    x = synth.make_activation(w)
    p = synth.make_weight_nvfp4(w)
    return x.to(dev()), p.codes.to(dev()), p.sf.to(dev()), torch.tensor([p.g], dtype=torch.float32, device=dev())


def test_noalloc_matches_the_allocating_layer_on_consecutive_calls():
    for i, (name, M, N, K, x_dt, o_dt, swiglu, mt, extra) in enumerate(CALLS):
        x, cd, sd, gs = _inputs(M, N, K, x_dt, swiglu, 40 + i)
        g = torch.Generator().manual_seed(i)
        pre = (torch.rand(K, generator=g) + 0.5).to(dev()) if extra else None
        bias = torch.randn(N, generator=g).to(dev()) if extra else None
        tdt = synth.TORCH_DTYPE[o_dt]
        full = torch.full((M, N + 8), 7, dtype=tdt, device=dev())
        out = full[:, :N]
        say(f"cr_linear_nvfp4_noalloc call {i + 1} ({name}): M={M} N={N} K={K} swiglu={swiglu} max_tile={mt}")
        rbl.cr_linear_nvfp4_noalloc(x, K, swiglu, cd, sd, gs, out, max_tile_bytes=mt, pre_scale=pre, bias=bias)
        say(f"cr_linear_nvfp4 reference for call {i + 1}")
        ref = rbl.linear_nvfp4(x, cd, sd, gs, K, out_dtype=tdt, swiglu=swiglu, pre_scale=pre, bias=bias)
        torch.cuda.synchronize()
        assert (full[:, N:] == 7).all(), "columns past N were written"
        assert torch.equal(out, ref), f"call {i + 1} ({name}) differs from cr_linear_nvfp4"


def test_noalloc_refuses_layers_beyond_the_scratch():
    """Host-side checks only: each call returns before any launch."""
    L = rbl.lib()
    A = 0x10000                     # a 256-byte aligned address that is never dereferenced
    stream = torch.cuda.current_stream().cuda_stream
    # QKV at M = 19989: the S8 activation alone is 107 MB
    assert L.cr_linear_nvfp4_noalloc(A, rbl.CR_BF16, 5376, 0, 19989, 5376, None, A, 2688, A, 336, A, 21504, None,
                                     A, rbl.CR_BF16, 21504, 0, 0, stream) == 4
    # an explicit tile bound whose two tiles do not fit beside the activation
    assert L.cr_linear_nvfp4_noalloc(A, rbl.CR_BF16, 5376, 0, 4096, 5376, None, A, 2688, A, 336, A, 21504, None,
                                     A, rbl.CR_BF16, 21504, 64 << 20, 0, stream) == 4
    # an empty batch is a valid call that enqueues nothing
    assert L.cr_linear_nvfp4_noalloc(None, rbl.CR_BF16, 5376, 0, 0, 5376, None, A, 2688, A, 336, A, 21504, None,
                                     None, rbl.CR_BF16, 21504, 0, 0, stream) == 0
