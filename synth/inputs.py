"""Seeded synthetic inputs for the rotated W8A8 linear layer.

This module is shared by the tests, the benchmark and the smoke check.  It holds no part
of the layer's own arithmetic (no rotation, no row quantization, no NVFP4 decode, no
GEMM): it only draws random numbers and packs a synthetic NVFP4 checkpoint, the way a
model's weights would have been quantized before the layer ever sees them.

Workloads (shapes from the modelpad.app MiniMax H3 explainer, parameter table of one
block: qkv_proj [21504, 5376], out_proj [5376, 7168] and the SwiGLU MLP with fc1
[28672, 5376] / fc2 [5376, 14336]; M = 19989 tokens and the K > 16384 streaming case from the "Load ConvRot
DiT and Load ConvRot CLIP" bullet of the ComfyUI Turing Utils README).  The pages measure
on real H3 NVFP4 weights with synthetic activations; real weights are not available, so
W = 0.02 * N(0, 1) encoded to NVFP4 stands in for them.

Recipe (every draw in float32 on the CPU, then one round-to-nearest-even cast):
  * config i (0-based) uses seed s = i; activations, weights, row/channel selections and
    padding garbage use separate generators seeded s, s + 1000, s + 2000 and s + 3000;
  * activations ~ N(0, 1); the QKV configs scale 1% of the channels (the first
    round(0.01 K) of a random permutation) by 20 before the cast (outlier channels);
  * the long-K config zeroes 2% of the rows and scales another disjoint 2% by 1e-4;
  * weights = 0.02 * N(0, 1), NVFP4-encoded as described in ``nvfp4_encode``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

DT_BF16, DT_FP16, DT_FP32, DT_I32 = 0, 1, 2, 3
TORCH_DTYPE = {DT_BF16: torch.bfloat16, DT_FP16: torch.float16, DT_FP32: torch.float32,
               DT_I32: torch.int32}
DTYPE_NAME = {DT_BF16: "bf16", DT_FP16: "fp16", DT_FP32: "fp32", DT_I32: "i32"}


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int                     # logical K (F, the SwiGLU half width, when swiglu)
    x_dtype: int
    out_dtypes: tuple
    seed: int
    swiglu: bool = False
    outlier_frac: float = 0.0  # fraction of channels scaled by outlier_scale
    outlier_scale: float = 20.0
    zero_row_frac: float = 0.0
    tiny_row_frac: float = 0.0
    tiny_row_scale: float = 1e-4
    note: str = field(default="", compare=False)

    @property
    def K_pad(self) -> int:
        return 256 * ((self.K + 255) // 256)

    @property
    def gemm_ops(self) -> int:
        return 2 * self.M * self.N * self.K_pad


WORKLOADS = {
    "tiny": Workload("tiny", 64, 256, 512, DT_BF16, (DT_BF16,), 0,
                     note="X[64,512] bf16, W[256,512] NVFP4"),
    "qkv_m4096": Workload("qkv_m4096", 4096, 21504, 5376, DT_BF16, (DT_BF16,), 1,
                          outlier_frac=0.01, note="qkv_proj [21504,5376] at M=4096"),
    "qkv": Workload("qkv", 19989, 21504, 5376, DT_BF16, (DT_BF16,), 2,
                    outlier_frac=0.01, note="qkv_proj [21504,5376] at M=19989"),
    "ffn_down": Workload("ffn_down", 19989, 5376, 14336, DT_BF16, (DT_BF16,), 3, swiglu=True,
                         note="SwiGLU + fc2 [5376,14336] at M=19989, H[19989,28672]"),
    "longk": Workload("longk", 8192, 5000, 20000, DT_FP16, (DT_FP16, DT_FP32), 4,
                      zero_row_frac=0.02, tiny_row_frac=0.02,
                      note="K=20000 (padded 20224, two-pass), N=5000 tail, fp16 in"),
    # the block's other linear layers (same kernels at new shapes)
    "out_proj": Workload("out_proj", 19989, 5376, 7168, DT_BF16, (DT_BF16,), 5,
                         note="out_proj [5376,7168] at M=19989"),
    "ffn_up": Workload("ffn_up", 19989, 28672, 5376, DT_BF16, (DT_BF16,), 6,
                       note="fc1 [28672,5376] at M=19989"),
    # a short batch of the same QKV layer: the shape where the weight decode dominates
    "qkv_m128": Workload("qkv_m128", 128, 21504, 5376, DT_BF16, (DT_BF16,), 7,
                         outlier_frac=0.01, note="qkv_proj [21504,5376] at M=128"),
}

# The MLP of one block as a chain: fc1 (ffn_up) writes H [M, 28672] in bf16, which the
# FFN-down layer reads through its fused SwiGLU.
MLP_CHAIN = ("ffn_up", "ffn_down")


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def round_up(v: int, m: int) -> int:
    return ((v + m - 1) // m) * m


def make_activation(w: Workload) -> torch.Tensor:
    """Activation X[M, K] (or H[M, 2F] for SwiGLU) in w.x_dtype, CPU tensor."""
    cols = 2 * w.K if w.swiglu else w.K
    x = torch.randn(w.M, cols, generator=_gen(w.seed), dtype=torch.float32)
    sel = _gen(w.seed + 2000)
    if w.outlier_frac > 0:
        n_out = round(w.outlier_frac * cols)
        ch = torch.randperm(cols, generator=sel)[:n_out]
        x[:, ch] *= w.outlier_scale
    if w.zero_row_frac > 0 or w.tiny_row_frac > 0:
        n_zero = round(w.zero_row_frac * w.M)
        n_tiny = round(w.tiny_row_frac * w.M)
        perm = torch.randperm(w.M, generator=sel)
        x[perm[:n_zero]] = 0.0
        x[perm[n_zero:n_zero + n_tiny]] *= w.tiny_row_scale
    return x.to(TORCH_DTYPE[w.x_dtype])


def special_rows(w: Workload):
    """(zero_rows, tiny_rows) index tensors of the long-K recipe, else empty tensors."""
    cols = 2 * w.K if w.swiglu else w.K
    sel = _gen(w.seed + 2000)
    if w.outlier_frac > 0:
        torch.randperm(cols, generator=sel)
    if w.zero_row_frac > 0 or w.tiny_row_frac > 0:
        n_zero = round(w.zero_row_frac * w.M)
        n_tiny = round(w.tiny_row_frac * w.M)
        perm = torch.randperm(w.M, generator=sel)
        return perm[:n_zero].clone(), perm[n_zero:n_zero + n_tiny].clone()
    e = torch.empty(0, dtype=torch.int64)
    return e, e


def make_weight_f32(w: Workload) -> torch.Tensor:
    """Dense float32 weight [N, K] = 0.02 * N(0, 1) (before NVFP4 encoding)."""
    return 0.02 * torch.randn(w.N, w.K, generator=_gen(w.seed + 1000), dtype=torch.float32)


# ----------------------------------------------------------------- NVFP4 packing ----

# E2M1 magnitudes by 3-bit code, and the decision points between neighbours.  A value
# exactly on a decision point goes to the neighbour with the even code.
_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


@dataclass
class NVFP4Weight:
    codes: torch.Tensor   # uint8 [N, ld_codes]; byte k//2 of a row holds element k, low nibble = even k
    sf: torch.Tensor      # uint8 [N, ld_sf]; E4M3 scale of the 16-element block k//16
    g: float              # fp32 global scale
    K: int

    @property
    def N(self) -> int:
        return self.codes.shape[0]

    @property
    def ld_codes(self) -> int:
        return self.codes.shape[1]

    @property
    def ld_sf(self) -> int:
        return self.sf.shape[1]


def nvfp4_encode(w: torch.Tensor, *, ld_codes: int | None = None, ld_sf: int | None = None,
                 garbage_seed: int | None = None) -> NVFP4Weight:
    """Pack a float32 [N, K] weight as NVFP4 with deterministic rounding.

    g = amax / (6 * 448) (1 if the tensor is zero); per 16-element block the E4M3 scale is
    the round-to-nearest-even E4M3 value of bamax / (6 g), saturated at 448; each element
    is the nearest E2M1 value of x / (scale * g), ties to the even code.  Bytes and
    nibbles past the logical K (row padding) are filled with random garbage when
    ``garbage_seed`` is given, else zero.
    """
    w = w.to(torch.float32)
    N, K = w.shape
    nb = (K + 15) // 16
    need_codes = (K + 1) // 2
    ld_codes = ld_codes if ld_codes is not None else round_up(need_codes, 16)
    ld_sf = ld_sf if ld_sf is not None else round_up(nb, 16)
    assert ld_codes >= need_codes and ld_sf >= nb

    amax = float(w.abs().max()) if w.numel() else 0.0
    g = torch.tensor(amax, dtype=torch.float32) / torch.tensor(6.0 * 448.0, dtype=torch.float32)
    if amax == 0.0:
        g = torch.tensor(1.0, dtype=torch.float32)
    wp = torch.zeros(N, nb * 16, dtype=torch.float32)
    wp[:, :K] = w
    blocks = wp.view(N, nb, 16)
    bamax = blocks.abs().amax(dim=-1)
    req = torch.clamp(bamax / (6.0 * g), max=448.0)
    sf8 = req.to(torch.float8_e4m3fn)
    sdec = sf8.to(torch.float32)
    denom = (sdec * g).unsqueeze(-1)
    safe = torch.where(denom > 0, denom, torch.ones_like(denom))
    x = blocks / safe
    mag = x.abs()
    code = torch.zeros_like(mag, dtype=torch.uint8)
    for i, t in enumerate(_E2M1_MID):
        up = (mag > t) if (i % 2 == 0) else (mag >= t)   # tie -> even code (i+1 even iff i odd)
        code += up.to(torch.uint8)
    code = torch.where((x < 0) & (code > 0), code | 8, code)
    code = torch.where(denom > 0, code, torch.zeros_like(code))
    code = code.view(N, nb * 16)

    lo = code[:, 0::2]
    hi = code[:, 1::2]
    packed = (lo | (hi << 4)).to(torch.uint8)            # [N, nb*8]
    codes = torch.zeros(N, ld_codes, dtype=torch.uint8)
    ncopy = min(packed.shape[1], ld_codes)
    codes[:, :ncopy] = packed[:, :ncopy]
    sf = torch.zeros(N, ld_sf, dtype=torch.uint8)
    sf[:, :nb] = sf8.view(torch.uint8)

    if garbage_seed is not None:
        gg = _gen(garbage_seed)
        junk_c = torch.randint(0, 256, (N, ld_codes), generator=gg, dtype=torch.int32).to(torch.uint8)
        junk_s = torch.randint(0, 256, (N, ld_sf), generator=gg, dtype=torch.int32).to(torch.uint8)
        codes[:, need_codes:] = junk_c[:, need_codes:]
        if K % 2 == 1:  # high nibble of the last used byte is padding
            last = need_codes - 1
            codes[:, last] = (codes[:, last] & 0x0F) | (junk_c[:, last] & 0xF0)
        sf[:, nb:] = junk_s[:, nb:]
    return NVFP4Weight(codes=codes, sf=sf, g=float(g), K=K)


def raw_nvfp4(N: int, K: int, seed: int, *, ld_codes: int | None = None, ld_sf: int | None = None,
              g: float = 0.0137, uniform_rows: bool = True) -> NVFP4Weight:
    """NVFP4 bytes drawn directly, not through an encoder: every code byte uniformly random
    (so all 16 nibbles appear, -0 included), every block-scale byte a finite E4M3 byte (all
    but 0x7F and 0xFF), and random garbage in the row padding of both arrays (NaN scale bytes
    included there).  With ``uniform_rows`` the first 254 rows each use one scale byte for
    the whole row, one row per finite byte in byte order; the remaining rows take the finite
    bytes in seeded shuffles, so every byte occurs in any 254 consecutive scale slots."""
    g_np = _gen(seed)
    nb = (K + 15) // 16
    ld_codes = ld_codes if ld_codes is not None else round_up((K + 1) // 2, 16)
    ld_sf = ld_sf if ld_sf is not None else nb
    codes = torch.randint(0, 256, (N, ld_codes), generator=g_np, dtype=torch.int32).to(torch.uint8)
    sf = torch.randint(0, 256, (N, ld_sf), generator=g_np, dtype=torch.int32).to(torch.uint8)
    finite = torch.tensor([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=torch.uint8)
    n_uni = min(N, 254) if uniform_rows else 0
    if n_uni:
        sf[:n_uni, :nb] = finite[:n_uni, None]
    rest = N - n_uni
    if rest:
        reps = -(-(rest * nb) // 254)
        pool = torch.cat([finite[torch.randperm(254, generator=g_np)] for _ in range(reps)])
        sf[n_uni:, :nb] = pool[:rest * nb].view(rest, nb)
    return NVFP4Weight(codes=codes, sf=sf, g=float(torch.tensor(g, dtype=torch.float32)), K=K)


def make_weight_nvfp4(w: Workload, **kw) -> NVFP4Weight:
    kw.setdefault("garbage_seed", w.seed + 3000)
    return nvfp4_encode(make_weight_f32(w), **kw)


def bits_u16(t: torch.Tensor):
    """numpy uint16 view of a bf16/fp16 CPU tensor (bit patterns)."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def sample_rows(M: int, n: int, seed: int, must: torch.Tensor | None = None) -> torch.Tensor:
    """Sorted seeded sample of n rows, always with the last min(M, 32) rows (the M tail)
    and every row in ``must``."""
    g = _gen(seed + 4000)
    n = min(n, M)
    pick = torch.randperm(M, generator=g)[:n]
    tail = torch.arange(max(0, M - 32), M)
    parts = [pick, tail]
    if must is not None and must.numel():
        parts.append(must.to(torch.int64))
    return torch.unique(torch.cat(parts)).sort().values


__all__ = ["Workload", "WORKLOADS", "MLP_CHAIN", "make_activation", "make_weight_f32", "make_weight_nvfp4",
           "nvfp4_encode", "raw_nvfp4", "NVFP4Weight", "special_rows", "sample_rows", "bits_u16",
           "DT_BF16", "DT_FP16", "DT_FP32", "DT_I32", "TORCH_DTYPE", "DTYPE_NAME", "round_up"]
