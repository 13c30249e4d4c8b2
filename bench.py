#!/usr/bin/env python3
"""Benchmark of the rotated W8A8 NVFP4 linear layer on one MI355X.

One step = the QKV projection layer (qkv_proj [21504, 5376]) and the FFN-down layer with
fused SwiGLU (fc2 [5376, 14336], H [19989, 28672]) at M = 19989 tokens, each one call of the
product entry point cr_linear_nvfp4 (activation preparation, NVFP4 weight preparation of each
chunk, INT8 MFMA GEMM with the row-scale epilogue, all on the calling stream).  Inputs are
seeded synthetic data resident in HBM before timing starts.  Staging the weight chunks on a
second stream (the pages' overlap) measures slower on this chip; --two-stream times that
schedule for value instead, and the JSON reports the other schedule apart from value.

Prints one JSON line: ms/layer (mean over the two layers of the product call, HIP events on
the calling stream), the per-kernel split of the same layers from a mirror of the call made
of the component calls (each launch between events on its own stream), the GEMM roofline
(INT8 MFMA peak), each kernel timed alone (preparation rates against the HBM peak and a
measured device copy; the weight preparation also against its vector-issue roofline), the
expanded-S8 control, the pages' 16 MiB staging bound, the other configurations (tiny, QKV at
M = 4096, long K with fp16 and fp32 outputs), the block's other shapes, short batches
(decode-inside-GEMM), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms/layer and INT8 TOPS (fraction of peak), QKV and FFN-down at M=19989"
PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 MFMA, TOP/s
PEAK_FP6_TOPS = 10100.0      # MI355X dense FP6 / FP4 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
BT = 2                       # CR_FLAG_BLOCK_TRANSPOSED: the order cr_linear_nvfp4 uses inside
# Decode-inside-GEMM: vector instructions per weight element at the minimum (decode: one
# conversion per two elements and two multiplies; rotation: 8 butterfly adds; quantization:
# multiply, rounding add and 3/4 of a byte permute) and the chip's vector issue peak with one
# fp32 operation per lane per clock (256 CUs x 64 lanes x 2.4 GHz; no packed math).
FUSED_VALU_PER_ELEM = 13.25
PEAK_VALU_TOPS = 39.3
# NVFP4 weight preparation, vector instructions per weight element at the minimum: decode 2.5,
# rotation 8, row maximum 0.5 (v_max3), quantization 2.75; weight rows streamed twice (K_pad > 32768)
# decode and rotate again (11 + 13.25).
WEIGHT_VALU_PER_ELEM = {False: 13.75, True: 24.25}
GEMM_SOURCES = ["rotated_bit_linear_amd/csrc/gemm_s8.hip", "rotated_bit_linear_amd/csrc/gemm_common.hpp"]
PMC_PROFILE = os.path.join(ROOT, "profiles", "gemm_s8_qkv_m19989_hbm_counters.md")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads", default="qkv,ffn_down")
    ap.add_argument("--next-shapes", default="out_proj,ffn_up,qkv+pre_bias",
                    help="other linear shapes of the block, reported apart from value ('' = none); "
                         "name+pre_bias adds a channel pre-scale and a bias")
    ap.add_argument("--short-batches", default="1,16,64,128",
                    help="activation rows of the short-batch (decode-inside-GEMM) lines; empty: none")
    ap.add_argument("--max-tile-bytes", type=int, default=0, help="0 = library default")
    ap.add_argument("--bounded-tile-mib", type=int, default=16,
                    help="also time the layers with S8 weight tiles bounded by this many MiB (0: skip)")
    ap.add_argument("--w4a8", default="qkv,ffn_down",
                    help="layers timed through the W4A8 variant, apart from value ('' = none)")
    ap.add_argument("--w4a4", default="qkv,ffn_down",
                    help="layers timed through the W4A4 variant, apart from value ('' = none)")
    ap.add_argument("--configs", default="tiny,qkv_m4096,longk",
                    help="the other configurations, reported apart from value ('' = none)")
    ap.add_argument("--two-stream", action="store_true",
                    help="stage weight tiles on a second stream (the pages' overlap) for value; by default "
                         "they are staged on the calling stream, which is faster on this chip")
    ap.add_argument("--no-stream-compare", action="store_true",
                    help="skip the line that times the other staging schedule")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=8192)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration) and exit")
    ap.add_argument("--json-out", default="")
    return ap.parse_args()


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(launch_shape):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary, or None if
    the GEMM source or the launch shape (M, N, K_pad) changed since the counters were taken."""
    if not os.path.exists(PMC_PROFILE):
        return None
    txt = open(PMC_PROFILE).read()
    m_hash = re.search(r"gemm_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_bytes = re.search(r"hbm_bytes_per_launch_calibrated:\s*([0-9.eE+]+)", txt)
    m_shape = re.search(r"launch_shape_m_n_kpad:\s*(\d+)\s+(\d+)\s+(\d+)", txt)
    if not (m_hash and m_bytes and m_shape) or m_hash.group(1) != gemm_source_hash():
        return None
    if tuple(int(v) for v in m_shape.groups()) != tuple(launch_shape):
        return None
    return float(m_bytes.group(1))


class Layer:
    def __init__(self, name, torch, rbl, synth, dev, max_tile_bytes, pre_bias=False, out_dtype=None):
        """pre_bias: also apply a channel pre-scale [K] and a bias [N] (seeded); out_dtype:
        one of the workload's output dtypes (default: its first)."""
        w = synth.WORKLOADS[name]
        odt = w.out_dtypes[0] if out_dtype is None else out_dtype
        suffix = "" if out_dtype is None else "_out_" + synth.DTYPE_NAME[odt]
        self.name, self.w = (name + ("_prescale_bias" if pre_bias else "") + suffix), w
        self.max_tile_bytes = max_tile_bytes
        t0 = time.perf_counter()
        x = synth.make_activation(w)
        p = synth.make_weight_nvfp4(w)
        self.host_x, self.host_p = x, p
        self.x = x.to(dev)
        self.codes, self.sf = p.codes.to(dev), p.sf.to(dev)
        self.g = torch.tensor([p.g], dtype=torch.float32, device=dev)
        kp = w.K_pad
        # the chunking cr_linear_nvfp4 uses on this device, mirrored with component calls;
        # no chunks means the short-batch path (the weight decoded inside the GEMM)
        self.R, self.nchunks = rbl.cr_linear_nvfp4_plan(w.M, w.N, w.K, max_tile_bytes)
        self.fused = self.nchunks == 0
        if self.fused:
            self.R = w.N
        self.n_launch = max(self.nchunks, 1)          # GEMM launches per layer
        self.chunks = [(n0, min(self.R, w.N - n0)) for n0 in range(0, w.N, self.R)]
        ntiles = 0 if self.fused else (2 if self.nchunks > 1 else 1)
        self.x_s8 = torch.empty(w.M, kp, dtype=torch.int8, device=dev)
        self.x_scale = torch.empty(w.M, dtype=torch.float32, device=dev)
        self.w_s8 = [torch.empty(self.R, kp, dtype=torch.int8, device=dev) for _ in range(ntiles)]
        self.w_scale = [torch.empty(self.R, dtype=torch.float32, device=dev) for _ in range(ntiles)]
        self.out = torch.empty(w.M, w.N, dtype=synth.TORCH_DTYPE[odt], device=dev)
        self.out_prod = torch.empty_like(self.out)      # the product call's output
        self.ws = torch.empty(max(1, rbl.cr_linear_nvfp4_workspace_bytes(w.M, w.N, w.K, max_tile_bytes)),
                              dtype=torch.uint8, device=dev)
        self.pre = self.bias = None
        if pre_bias:
            g = torch.Generator().manual_seed(w.seed + 5000)
            self.pre = (torch.rand(w.K, generator=g) * 1.5 + 0.5).to(dev)
            self.bias = torch.randn(w.N, generator=g).to(dev)
        self.gen_s = time.perf_counter() - t0
        es = self.x.element_size()
        cols = 2 * w.K if w.swiglu else w.K
        self.act_bytes = w.M * cols * es + w.M * kp + 4 * w.M
        self.w_bytes = w.N * ((w.K + 1) // 2) + w.N * ((w.K + 15) // 16) + 4 + w.N * kp + 4 * w.N
        self.gemm_ops = 2 * w.M * w.N * kp
        self.n_events = 3 + 4 * self.n_launch


def run_product(L, rbl, s_main, s_aux):
    """One call of the product entry point (cr_linear_nvfp4, or cr_linear_nvfp4_ex with a
    pre-scale and a bias) on the main stream, weight tiles staged on s_aux."""
    rbl.cr_linear_nvfp4(L.x, L.w.K, L.w.swiglu, L.codes, L.sf, L.g, L.out_prod, L.ws, L.max_tile_bytes,
                        stream=s_main, aux_stream=s_aux, pre_scale=L.pre, bias=L.bias)


def time_product(torch, rbl, layers, K, W, s_main, s_aux):
    """W untimed steps, then K timed steps of the product call on every layer: per-layer
    per-step ms (events recorded on the calling stream around each call), ms per step over
    the whole loop, and the host wall time of the loop."""
    mk = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    evs = [[(mk(), mk()) for _ in layers] for _ in range(K)]
    print(f"bench: warmup {W} steps of cr_linear_nvfp4 on {[L.name for L in layers]}", file=sys.stderr, flush=True)
    for _ in range(W):
        for L in layers:
            run_product(L, rbl, s_main, s_aux)
    torch.cuda.synchronize()
    print(f"bench: timing {K} steps of cr_linear_nvfp4", file=sys.stderr, flush=True)
    start, end = mk(), mk()
    t0 = time.perf_counter()
    start.record(s_main)
    for k in range(K):
        for li, L in enumerate(layers):
            evs[k][li][0].record(s_main)
            run_product(L, rbl, s_main, s_aux)
            evs[k][li][1].record(s_main)
    end.record(s_main)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0
    per_layer = [[evs[k][li][0].elapsed_time(evs[k][li][1]) for k in range(K)] for li in range(len(layers))]
    return per_layer, start.elapsed_time(end) / K, wall_ms


def product_stats(times):
    t = sorted(times)
    return {"ms": round(sum(t) / len(t), 4), "ms_median": round(t[len(t) // 2], 4), "ms_min": round(t[0], 4)}


def run_layer(L, rbl, s_main, s_aux, ev):
    """The component mirror of the layer, as cr_linear_nvfp4 runs it.  Without s_aux every
    launch goes in order on the main stream.  With s_aux: activation prep (main stream) while
    chunk 0 of the weight is prepared (second stream); GEMM of chunk c on the main stream
    while chunk c+1 is prepared; a weight tile is refilled only after the GEMM that read it;
    a weight of one chunk is staged on the main stream.
    ev: 3 + 4 * nchunks events: start, act begin/end, then per chunk prep begin/end and
    GEMM begin/end."""
    w = L.w
    if L.fused:                                       # short batch: the weight decoded in the GEMM
        ev[0].record(s_main)
        if L.pre is not None:
            rbl.cr_quant_act_ex(L.x, w.K, w.swiglu, L.pre, L.x_s8, L.x_scale, BT, stream=s_main)
        elif w.swiglu:
            rbl.cr_quant_act_swiglu(L.x, w.K, L.x_s8, L.x_scale, BT, stream=s_main)
        else:
            rbl.cr_quant_act(L.x, w.K, L.x_s8, L.x_scale, BT, stream=s_main)
        ev[1].record(s_main)
        ev[3].record(s_main)                          # no separate weight preparation
        ev[4].record(s_main)
        ev[5].record(s_main)
        rbl.cr_gemm_nvfp4_fused(L.x_s8, L.x_scale, L.codes, L.sf, L.g, None, w.K, L.out, bias=L.bias, flags=BT,
                                stream=s_main)
        ev[6].record(s_main)
        ev[2].record(s_main)
        return
    if L.nchunks < 2:
        s_aux = None                                  # a single chunk is staged on the main stream
    sw = s_aux if s_aux is not None else s_main
    ev[0].record(s_main)
    if s_aux is not None:
        s_aux.wait_event(ev[0])
    if L.pre is not None:
        rbl.cr_quant_act_ex(L.x, w.K, w.swiglu, L.pre, L.x_s8, L.x_scale, BT, stream=s_main)
    elif w.swiglu:
        rbl.cr_quant_act_swiglu(L.x, w.K, L.x_s8, L.x_scale, BT, stream=s_main)
    else:
        rbl.cr_quant_act(L.x, w.K, L.x_s8, L.x_scale, BT, stream=s_main)
    ev[1].record(s_main)
    for c, (n0, r) in enumerate(L.chunks):
        t = c % 2
        e = 3 + 4 * c
        if c >= 2 and s_aux is not None:
            s_aux.wait_event(ev[e - 8 + 3])           # GEMM of chunk c-2 read this tile
        ev[e].record(sw)
        rbl.cr_prep_weight_nvfp4(L.codes[n0:n0 + r], L.sf[n0:n0 + r], L.g, w.K, L.w_s8[t][:r],
                                 L.w_scale[t][:r], BT, stream=sw)
        ev[e + 1].record(sw)
        if s_aux is not None:
            s_main.wait_event(ev[e + 1])
        ev[e + 2].record(s_main)
        if L.bias is not None:
            rbl.cr_gemm_s8_rowscale_bias(L.x_s8, L.x_scale, L.w_s8[t][:r], L.w_scale[t][:r], L.bias[n0:n0 + r],
                                         L.out[:, n0:n0 + r], stream=s_main)
        else:
            rbl.cr_gemm_s8_rowscale(L.x_s8, L.x_scale, L.w_s8[t][:r], L.w_scale[t][:r],
                                    L.out[:, n0:n0 + r], stream=s_main)
        ev[e + 3].record(s_main)
    ev[2].record(s_main)


def time_layers(torch, rbl, layers, K, W, s_main, s_aux):
    """W untimed steps, then K timed steps over `layers`; per-step per-layer events,
    ms per step (HIP events on the main stream) and the host wall time of the loop."""
    mk = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731
    evs = [[[mk() for _ in range(L.n_events)] for L in layers] for _ in range(K)]
    scratch = [[mk() for _ in range(L.n_events)] for L in layers]
    print(f"bench: warmup {W} steps of {[L.name for L in layers]}", file=sys.stderr, flush=True)
    for _ in range(W):
        for li, L in enumerate(layers):
            run_layer(L, rbl, s_main, s_aux, scratch[li])
    torch.cuda.synchronize()
    print(f"bench: timing {K} steps", file=sys.stderr, flush=True)
    start, end = mk(), mk()
    t0 = time.perf_counter()
    start.record(s_main)
    for k in range(K):
        for li, L in enumerate(layers):
            run_layer(L, rbl, s_main, s_aux, evs[k][li])
    end.record(s_main)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1000.0
    return evs, start.elapsed_time(end) / K, wall_ms


def layer_stats(L, ev_steps):
    """Per-layer figures from the events of each timed step (see run_layer)."""
    K = len(ev_steps)

    def mean(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in ev_steps) / K
    nc = L.n_launch
    t_layer = mean(0, 2)
    per_step = sorted(e[0].elapsed_time(e[2]) for e in ev_steps)
    t_act = mean(0, 1)
    t_w = sum(mean(3 + 4 * c, 4 + 4 * c) for c in range(nc))
    g_launch = [mean(5 + 4 * c, 6 + 4 * c) for c in range(nc)]
    t_g = sum(g_launch)
    return {
        "M": L.w.M, "N": L.w.N, "K": L.w.K, "K_pad": L.w.K_pad, "swiglu": L.w.swiglu,
        "weight_chunks": L.nchunks, "rows_per_chunk": L.R,
        "path": "decode-inside-GEMM" if L.fused else "staged",
        "ms": round(t_layer, 4),
        "ms_median": round(per_step[K // 2], 4),
        "ms_min": round(per_step[0], 4),
        "gemm_ms": round(t_g, 4),
        "gemm_launch_ms": [round(v, 4) for v in g_launch],
        "gemm_tops": round(L.gemm_ops / (t_g * 1e-3) / 1e12, 1),
        "gemm_frac_peak": round(L.gemm_ops / (t_g * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
        "layer_tops": round(L.gemm_ops / (t_layer * 1e-3) / 1e12, 1),
        "act_prep_ms": round(t_act, 4),
        "act_prep_gbs": round(L.act_bytes / (t_act * 1e-3) / 1e9, 1),
        "weight_prep_ms": round(t_w, 4),
        "weight_prep_gbs": round(L.w_bytes / (t_w * 1e-3) / 1e9, 1) if t_w > 0 else None,
        "not_gemm_ms": round(t_layer - t_g, 4),
    }


def cpu_baseline(layers, sample_rows):
    """The CPU oracle, as it stands, on a bounded sample: the whole weight preparation
    (a fixed per-layer cost) plus activation preparation, int32 GEMM and epilogue on the
    first `sample_rows` rows, extrapolated linearly in M (rows are independent)."""
    import numpy as np

    import oracle
    import synth
    per_layer = []
    detail = {}
    t_all = time.perf_counter()
    for L in layers:
        w, p = L.w, L.host_p
        m = min(sample_rows, w.M)
        xs = L.host_x[:m]
        xb = xs.contiguous().numpy() if w.x_dtype == synth.DT_FP32 else synth.bits_u16(xs)
        t0 = time.perf_counter()
        qw, sw = oracle.prep_weight_nvfp4(p.codes.numpy(), p.sf.numpy(), p.g, w.K)
        t1 = time.perf_counter()
        qx, sx = oracle.quant_act(xb, w.x_dtype, w.K, swiglu=w.swiglu)
        acc = oracle.gemm_s8(qx, qw)
        oracle.epilogue(acc, sx, sw, w.out_dtypes[0])
        t2 = time.perf_counter()
        est = (t1 - t0) + (t2 - t1) * (w.M / m)
        per_layer.append(est)
        detail[L.name] = {"weight_prep_s": round(t1 - t0, 3), "rows": m, "rows_s": round(t2 - t1, 3),
                          "layer_s_extrapolated": round(est, 2)}
        del qw, qx, acc
    wall = time.perf_counter() - t_all
    return {
        "value": round(1000.0 * sum(per_layer) / len(per_layer), 1),
        "unit": "ms/layer",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"whole weight preparation + first {sample_rows} rows of activation prep, int32 GEMM "
                   f"and epilogue per layer, extrapolated linearly to M=19989; {wall:.1f} s of CPU work"),
        "detail": detail,
    }


def time_loop(torch, fn, stream, n=10, warm=2):
    """Mean ms of fn() over n back-to-back calls, HIP events on `stream`."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def copy_bandwidth(torch, stream) -> float:
    """GB/s (bytes read + written) of a plain 1 GiB device-to-device copy."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    ms = time_loop(torch, lambda: dst.copy_(src), stream, n=5)
    del src, dst
    return 2 * n / (ms * 1e-3) / 1e9


def short_batches(torch, rbl, synth, dev, s_main, rows_list, n=20):
    """The QKV weight [21504, 5376] at short batches: the layer as cr_linear_nvfp4 runs it
    (decode-inside-GEMM up to 64 rows, staged tiles above), the same call captured into a HIP
    graph and replayed, the staged components one after the other (activation prep,
    whole-weight prep, GEMM), and the fused GEMM with the weight's row maxima computed once,
    as for a fixed weight.  Returns the per-batch times and the
    fused kernel's vector-issue roofline at the smallest batch."""
    w = synth.WORKLOADS["qkv_m128"]
    p = synth.make_weight_nvfp4(w)
    x_all = synth.make_activation(synth.Workload("short", max(rows_list), w.N, w.K, w.x_dtype, w.out_dtypes,
                                                 w.seed, outlier_frac=w.outlier_frac)).to(dev)
    cd, sfd = p.codes.to(dev), p.sf.to(dev)
    gs = torch.tensor([p.g], dtype=torch.float32, device=dev)
    amax = torch.empty(w.N, dtype=torch.float32, device=dev)
    w_s8 = torch.empty(w.N, w.K_pad, dtype=torch.int8, device=dev)
    w_sc = torch.empty(w.N, dtype=torch.float32, device=dev)
    t_amax = time_loop(torch, lambda: rbl.cr_weight_amax_nvfp4(cd, sfd, gs, w.K, amax, stream=s_main), s_main, n=n)
    aux = torch.cuda.Stream()
    info = {"weight": "qkv_proj [21504, 5376] NVFP4", "weight_row_maxima_ms": round(t_amax, 4), "rows": {}}
    t_gemm_small = None
    for M in rows_list:
        x = x_all[:M]
        qx = torch.empty(M, w.K_pad, dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        y = torch.empty(M, w.N, dtype=torch.bfloat16, device=dev)
        y2 = torch.empty_like(y)
        ws = torch.empty(rbl.cr_linear_nvfp4_workspace_bytes(M, w.N, w.K), dtype=torch.uint8, device=dev)

        def layer():
            rbl.cr_linear_nvfp4(x, w.K, False, cd, sfd, gs, y, ws, stream=s_main, aux_stream=aux)

        def staged():
            rbl.cr_quant_act(x, w.K, qx, sx, BT, stream=s_main)
            rbl.cr_prep_weight_nvfp4(cd, sfd, gs, w.K, w_s8, w_sc, BT, stream=s_main)
            rbl.cr_gemm_s8_rowscale(qx, sx, w_s8, w_sc, y2, stream=s_main)

        def fused_gemm():
            rbl.cr_gemm_nvfp4_fused(qx, sx, cd, sfd, gs, amax, w.K, y2, flags=BT, stream=s_main)

        def fused_cached():
            rbl.cr_quant_act(x, w.K, qx, sx, BT, stream=s_main)
            fused_gemm()

        t_l, t_s = time_loop(torch, layer, s_main, n=n), time_loop(torch, staged, s_main, n=n)
        same_staged = torch.equal(y, y2)
        # the same layer call captured once into a HIP graph and replayed
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            rbl.cr_linear_nvfp4(x, w.K, False, cd, sfd, gs, y, ws, aux_stream=aux)
        t_gr = time_loop(torch, graph.replay, s_main, n=n)
        torch.cuda.synchronize()
        same_staged = same_staged and torch.equal(y, y2)
        del graph
        t_c, t_g = time_loop(torch, fused_cached, s_main, n=n), time_loop(torch, fused_gemm, s_main, n=n)
        torch.cuda.synchronize()
        same = same_staged and torch.equal(y, y2)
        if t_gemm_small is None:
            t_gemm_small = (M, t_g)
        info["rows"][str(M)] = {
            "path": "decode-inside-GEMM" if rbl.cr_linear_nvfp4_plan(M, w.N, w.K)[1] == 0 else "staged",
            "layer_ms": round(t_l, 4),
            "layer_graph_replay_ms": round(t_gr, 4),
            "staged_components_ms": round(t_s, 4),
            "fused_with_cached_row_maxima_ms": round(t_c, 4),
            "fused_gemm_ms": round(t_g, 4),
            "outputs_identical": bool(same),
        }
        del qx, sx, y, y2, ws
    M0, tg = t_gemm_small
    ops = FUSED_VALU_PER_ELEM * w.N * w.K_pad
    achieved = ops / (tg * 1e-3) / 1e12
    info["fused_roofline"] = {"kernel": f"gemm_nvfp4_fused (M={M0} N={w.N} K_pad={w.K_pad})", "bound": "alu",
                              "achieved": round(achieved, 2), "peak": PEAK_VALU_TOPS, "unit": "Tops/s",
                              "frac": round(achieved / PEAK_VALU_TOPS, 4),
                              "per_element_ops": FUSED_VALU_PER_ELEM}
    return info


def w4a8_layers(torch, rbl, synth, dev, names, s_main, n=20):
    """The W4A8 variant at the metric's shapes: the weight (0.02 * N(0, 1), dense fp32) prepared
    once to rotated 4-bit rows (block-transposed order, timed apart as the offline step), then
    the layer call cr_linear_w4a8 and its GEMM alone; outputs of the layer and of activation
    prep + GEMM must agree."""
    info = {}
    for name in names:
        w = synth.WORKLOADS[name]
        x = synth.make_activation(w).to(dev)
        wf = synth.make_weight_f32(w).to(dev)
        p = torch.empty(w.N, w.K_pad // 2, dtype=torch.uint8, device=dev)
        sw = torch.empty(w.N, dtype=torch.float32, device=dev)
        t_prep = time_loop(torch, lambda: rbl.cr_quant_weight_w4(wf, w.K, p, sw, BT, stream=s_main), s_main, n=3)
        del wf
        out = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev)
        out2 = torch.empty_like(out)
        ws = torch.empty(rbl.cr_linear_w4a8_workspace_bytes(w.M, w.K), dtype=torch.uint8, device=dev)
        qx = torch.empty(w.M, w.K_pad, dtype=torch.int8, device=dev)
        sx = torch.empty(w.M, dtype=torch.float32, device=dev)
        act = ((lambda: rbl.cr_quant_act_swiglu(x, w.K, qx, sx, BT, stream=s_main)) if w.swiglu else
               (lambda: rbl.cr_quant_act(x, w.K, qx, sx, BT, stream=s_main)))
        layer = lambda: rbl.cr_linear_w4a8(x, w.K, w.swiglu, p, sw, out, ws, flags=BT, stream=s_main)  # noqa: E731
        gemm = lambda: rbl.cr_gemm_s8s4_rowscale(qx, sx, p, sw, out2, stream=s_main)  # noqa: E731
        # the weight was just made on the host (the GPU idled): warm as long as the timed loop
        t_layer = time_loop(torch, layer, s_main, n=n, warm=n)
        act()
        t_gemm = time_loop(torch, gemm, s_main, n=n)
        torch.cuda.synchronize()
        if not torch.equal(out, out2):
            raise SystemExit(f"bench: cr_linear_w4a8 differs from activation prep + W4A8 GEMM on {name}")
        ops = 2 * w.M * w.N * w.K_pad
        info[name] = {
            "M": w.M, "N": w.N, "K": w.K, "K_pad": w.K_pad, "swiglu": w.swiglu,
            "layer_ms": round(t_layer, 4),
            "gemm_ms": round(t_gemm, 4),
            "gemm_tops": round(ops / (t_gemm * 1e-3) / 1e12, 1),
            "gemm_frac_peak": round(ops / (t_gemm * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
            "weight_bytes_packed": w.N * w.K_pad // 2,
            "offline_weight_prep_ms": round(t_prep, 4),
        }
        del x, p, sw, out, out2, ws, qx, sx
    return info


def w4a4_layers(torch, rbl, synth, dev, names, s_main, n=20):
    """The W4A4 variant at the metric's shapes: the weight prepared as for W4A8, then the layer
    call cr_linear_w4a4, its activation preparation and its GEMM alone; outputs of the layer
    and of activation prep + GEMM must agree."""
    info = {}
    for name in names:
        w = synth.WORKLOADS[name]
        x = synth.make_activation(w).to(dev)
        wf = synth.make_weight_f32(w).to(dev)
        p = torch.empty(w.N, w.K_pad // 2, dtype=torch.uint8, device=dev)
        sw = torch.empty(w.N, dtype=torch.float32, device=dev)
        rbl.cr_quant_weight_w4(wf, w.K, p, sw, BT, stream=s_main)
        torch.cuda.synchronize()
        del wf
        out = torch.empty(w.M, w.N, dtype=torch.bfloat16, device=dev)
        out2 = torch.empty_like(out)
        ws = torch.empty(rbl.cr_linear_w4a4_workspace_bytes(w.M, w.K), dtype=torch.uint8, device=dev)
        qx = torch.empty(w.M, w.K_pad // 2, dtype=torch.uint8, device=dev)
        sx = torch.empty(w.M, dtype=torch.float32, device=dev)
        act = lambda: rbl.cr_quant_act_w4(x, w.K, w.swiglu, qx, sx, BT, stream=s_main)  # noqa: E731
        layer = lambda: rbl.cr_linear_w4a4(x, w.K, w.swiglu, p, sw, out, ws, flags=BT, stream=s_main)  # noqa: E731
        gemm = lambda: rbl.cr_gemm_s4s4_rowscale(qx, sx, p, sw, out2, stream=s_main)  # noqa: E731
        # the weight was just made on the host (the GPU idled): warm as long as the timed loop
        t_layer = time_loop(torch, layer, s_main, n=n, warm=n)
        t_act = time_loop(torch, act, s_main, n=n)
        t_gemm = time_loop(torch, gemm, s_main, n=n)
        torch.cuda.synchronize()
        if not torch.equal(out, out2):
            raise SystemExit(f"bench: cr_linear_w4a4 differs from activation prep + W4A4 GEMM on {name}")
        del qx, ws
        # the same layer on the 6-bit matrix cores (codes as E2M3 fields): identical outputs
        wf = synth.make_weight_f32(w).to(dev)
        lf = 3 * w.K_pad                  # E2M3 fields: bytes per quad of rows
        p6 = torch.empty((w.N + 3) // 4, lf, dtype=torch.uint8, device=dev)
        sw6 = torch.empty(w.N, dtype=torch.float32, device=dev)
        rbl.cr_quant_weight_w4_e2m3(wf, w.K, p6, sw6, BT, stream=s_main)
        torch.cuda.synchronize()
        del wf
        out6 = torch.empty_like(out)
        ws6 = torch.empty(rbl.cr_linear_w4a4_e2m3_workspace_bytes(w.M, w.K), dtype=torch.uint8, device=dev)
        qx6 = torch.empty((w.M + 3) // 4, lf, dtype=torch.uint8, device=dev)
        act6 = lambda: rbl.cr_quant_act_w4_e2m3(x, w.K, w.swiglu, qx6, sx, BT, stream=s_main)  # noqa: E731
        layer6 = lambda: rbl.cr_linear_w4a4_e2m3(x, w.K, w.swiglu, p6, sw6, out6, ws6, flags=BT,  # noqa: E731
                                                 stream=s_main)
        gemm6 = lambda: rbl.cr_gemm_e2m3_rowscale(qx6, sx, p6, sw6, out2, stream=s_main)  # noqa: E731
        t_layer6 = time_loop(torch, layer6, s_main, n=n, warm=n)
        t_act6 = time_loop(torch, act6, s_main, n=n)
        t_gemm6 = time_loop(torch, gemm6, s_main, n=n)
        torch.cuda.synchronize()
        if not (torch.equal(out6, out) and torch.equal(out2, out)):
            raise SystemExit(f"bench: the E2M3 W4A4 layer differs from the nibble-form layer on {name}")
        ops = 2 * w.M * w.N * w.K_pad
        in_cols = 2 * w.K if w.swiglu else w.K
        act_bytes = w.M * (in_cols * x.element_size() + w.K_pad // 2 + 4)
        act6_bytes = w.M * (in_cols * x.element_size() + w.K_pad // 4 * 3 + 4)
        info[name] = {
            "M": w.M, "N": w.N, "K": w.K, "K_pad": w.K_pad, "swiglu": w.swiglu,
            "layer_ms": round(t_layer, 4),
            "act_prep_ms": round(t_act, 4),
            "act_prep_gbs": round(act_bytes / (t_act * 1e-3) / 1e9, 1),
            "gemm_ms": round(t_gemm, 4),
            "gemm_tops": round(ops / (t_gemm * 1e-3) / 1e12, 1),
            "gemm_frac_peak": round(ops / (t_gemm * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
            "e2m3": {
                "layer_ms": round(t_layer6, 4),
                "act_prep_ms": round(t_act6, 4),
                "act_prep_gbs": round(act6_bytes / (t_act6 * 1e-3) / 1e9, 1),
                "gemm_ms": round(t_gemm6, 4),
                "gemm_tops": round(ops / (t_gemm6 * 1e-3) / 1e12, 1),
                "gemm_frac_fp6_peak": round(ops / (t_gemm6 * 1e-3) / 1e12 / PEAK_FP6_TOPS, 4),
            },
        }
        del x, p, sw, out, out2, sx, p6, sw6, out6, ws6, qx6
    return info


def copy_calibration(mib: int):
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def alone_stats(torch, rbl, L, s_main, copy_gbs, n=10):
    """Each kernel of the layer alone on the main stream, and the expanded-S8 control (the
    whole weight prepared once outside timing, then activation prep + one full-N GEMM)."""
    w = L.w
    dev = L.x.device
    w_full = torch.empty(w.N, w.K_pad, dtype=torch.int8, device=dev)
    ws_full = torch.empty(w.N, dtype=torch.float32, device=dev)
    act = ((lambda: rbl.cr_quant_act_swiglu(L.x, w.K, L.x_s8, L.x_scale, BT, stream=s_main)) if w.swiglu else
           (lambda: rbl.cr_quant_act(L.x, w.K, L.x_s8, L.x_scale, BT, stream=s_main)))
    wprep = lambda: rbl.cr_prep_weight_nvfp4(L.codes, L.sf, L.g, w.K, w_full, ws_full, BT, stream=s_main)  # noqa: E731
    gemm = lambda: rbl.cr_gemm_s8_rowscale(L.x_s8, L.x_scale, w_full, ws_full, L.out, stream=s_main)  # noqa: E731
    t_a = time_loop(torch, act, s_main, n=n)
    t_w = time_loop(torch, wprep, s_main, n=n)
    t_g = time_loop(torch, gemm, s_main, n=n)
    t_x = time_loop(torch, lambda: (act(), gemm()), s_main, n=n)
    valu = w.N * w.K_pad * WEIGHT_VALU_PER_ELEM[w.K_pad > 32768] / (t_w * 1e-3) / 1e12
    out = {
        "act_prep_ms": round(t_a, 4),
        "act_prep_gbs": round(L.act_bytes / (t_a * 1e-3) / 1e9, 1),
        "act_prep_frac_hbm_peak": round(L.act_bytes / (t_a * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "act_prep_frac_copy": round(L.act_bytes / (t_a * 1e-3) / 1e9 / copy_gbs, 4),
        "weight_prep_ms": round(t_w, 4),
        "weight_prep_gbs": round(L.w_bytes / (t_w * 1e-3) / 1e9, 1),
        "weight_prep_frac_hbm_peak": round(L.w_bytes / (t_w * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "weight_prep_frac_copy": round(L.w_bytes / (t_w * 1e-3) / 1e9 / copy_gbs, 4),
        # the weight preparation is bound by vector issue, not bytes: its own roofline
        "weight_prep_valu_tops": round(valu, 2),
        "weight_prep_frac_valu_peak": round(valu / PEAK_VALU_TOPS, 4),
        "gemm_full_n_ms": round(t_g, 4),
        "gemm_full_n_tops": round(L.gemm_ops / (t_g * 1e-3) / 1e12, 1),
        "gemm_full_n_frac_peak": round(L.gemm_ops / (t_g * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
        "expanded_s8_control_ms": round(t_x, 4),
    }
    del w_full, ws_full
    return out


def check_product_equals_mirror(torch, L):
    torch.cuda.synchronize()
    if not torch.equal(L.out, L.out_prod):
        raise SystemExit(f"bench: cr_linear_nvfp4 differs from the component calls on {L.name}")


def measure_layers(torch, rbl, layers, K, W, s_main, s_aux):
    """The product call timed over K steps (per-layer figures and ms per step), then the
    component mirror over K steps for the per-kernel split; the two outputs must agree."""
    prod, ms_step, wall = time_product(torch, rbl, layers, K, W, s_main, s_aux)
    evs, mirror_step, _ = time_layers(torch, rbl, layers, K, W, s_main, s_aux)
    info = {}
    for li, L in enumerate(layers):
        check_product_equals_mirror(torch, L)
        ps = product_stats(prod[li])
        split = layer_stats(L, [evs[k][li] for k in range(K)])
        d = {k: split[k] for k in ("M", "N", "K", "K_pad", "swiglu", "weight_chunks", "rows_per_chunk", "path")}
        d.update(ps)
        d["layer_tops"] = round(L.gemm_ops / (ps["ms"] * 1e-3) / 1e12, 1)
        d["split"] = {k: v for k, v in split.items() if k not in d}
        d["split"]["component_mirror_ms"] = split["ms"]
        d["product_minus_mirror_ms"] = round(ps["ms"] - split["ms"], 4)
        info[L.name] = d
    return info, ms_step, wall, mirror_step


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: runs on one GPU only (the layer is data-parallel over tokens with no "
              "communication; multi-GPU sharding is not implemented). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return

    import torch

    import rotated_bit_linear_amd as rbl
    import synth

    dev = torch.device("cuda:0")
    rbl.lib()
    names = [n.strip() for n in args.workloads.split(",") if n.strip()]
    layers = []
    for n in names:
        print(f"bench: generating {n} ...", file=sys.stderr, flush=True)
        layers.append(Layer(n, torch, rbl, synth, dev, args.max_tile_bytes))
    torch.cuda.synchronize()

    s_main = torch.cuda.current_stream()
    s_aux = torch.cuda.Stream() if args.two_stream else None
    K, W = args.steps, args.warmup
    layer_info, ms_per_step, wall_ms, mirror_step = measure_layers(torch, rbl, layers, K, W, s_main, s_aux)

    print("bench: components alone and the expanded-S8 control", file=sys.stderr, flush=True)
    copy_gbs = copy_bandwidth(torch, s_main)
    for L in layers:
        layer_info[L.name]["alone"] = alone_stats(torch, rbl, L, s_main, copy_gbs)

    # the other staging schedule (the pages' second stream, or serial staging when value
    # uses the second stream), product call, same layers, reported apart from value
    other_staging = None
    if not args.no_stream_compare:
        alt = None if args.two_stream else torch.cuda.Stream()
        print(f"bench: the layers with weight tiles staged {'serially' if alt is None else 'on a second stream'}",
              file=sys.stderr, flush=True)
        k2 = max(5, K // 2)
        prod, _, _ = time_product(torch, rbl, layers, k2, W, s_main, alt)
        other_staging = {"weight_prep_stream": "second stream" if alt is not None else "calling stream (serial staging)",
                         "layers": {}}
        for li, L in enumerate(layers):
            check_product_equals_mirror(torch, L)
            st = product_stats(prod[li])
            st["vs_value_ms"] = round(st["ms"] - layer_info[L.name]["ms"], 4)
            other_staging["layers"][L.name] = st
        other_staging["value_ms_per_layer"] = round(
            sum(v["ms"] for v in other_staging["layers"].values()) / len(layers), 4)

    # the pages' bound on one S8 weight tile (16 MiB), same layers, product call, same staging as value
    staging = None
    if args.bounded_tile_mib > 0:
        mt = args.bounded_tile_mib << 20
        print(f"bench: the layers with S8 tiles bounded by {args.bounded_tile_mib} MiB", file=sys.stderr, flush=True)
        for L in layers:
            L.max_tile_bytes = mt
            L.ws = torch.empty(rbl.cr_linear_nvfp4_workspace_bytes(L.w.M, L.w.N, L.w.K, mt), dtype=torch.uint8,
                               device=dev)
        k2 = max(5, K // 2)
        prod, _, _ = time_product(torch, rbl, layers, k2, W, s_main, s_aux)
        staging = {"max_tile_bytes": mt, "layers": {}}
        for li, L in enumerate(layers):
            check_product_equals_mirror(torch, L)
            R, nch = rbl.cr_linear_nvfp4_plan(L.w.M, L.w.N, L.w.K, mt)
            st = product_stats(prod[li])
            st.update({"rows_per_chunk": R, "weight_chunks": nch, "workspace_bytes": L.ws.numel(),
                       "vs_default_bound_ms": round(st["ms"] - layer_info[L.name]["ms"], 4)})
            staging["layers"][L.name] = st
        staging["value_ms_per_layer"] = round(sum(v["ms"] for v in staging["layers"].values()) / len(layers), 4)
        for L in layers:
            L.max_tile_bytes = args.max_tile_bytes
            L.ws = torch.empty(1, dtype=torch.uint8, device=dev)

    # the other configurations (tiny, QKV at M = 4096, long K with both output dtypes):
    # product call + per-kernel split + each kernel alone, reported apart from `value`
    cfg_info = None
    cfgs = [c.strip() for c in args.configs.split(",") if c.strip()]
    if cfgs:
        extra = []
        for n in cfgs:
            w = synth.WORKLOADS[n]
            for odt in w.out_dtypes:
                print(f"bench: generating config {n} out={synth.DTYPE_NAME[odt]} ...", file=sys.stderr, flush=True)
                extra.append(Layer(n, torch, rbl, synth, dev, args.max_tile_bytes,
                                   out_dtype=odt if len(w.out_dtypes) > 1 else None))
        torch.cuda.synchronize()
        k2 = max(5, K // 2)
        cfg_info, _, _, _ = measure_layers(torch, rbl, extra, k2, W, s_main, s_aux)
        for L in extra:
            cfg_info[L.name]["note"] = L.w.note
            cfg_info[L.name]["alone"] = alone_stats(torch, rbl, L, s_main, copy_gbs)
        del extra

    # the block's other linear shapes (same kernels), timed the same way but apart from
    # `value`; the MLP chain is fc1 followed by the FFN-down layer
    next_info = None
    nxt = [n.strip() for n in args.next_shapes.split(",") if n.strip()]
    if nxt:
        extra = []
        for n in nxt:
            print(f"bench: generating {n} ...", file=sys.stderr, flush=True)
            base, _, opt = n.partition("+")
            extra.append(Layer(base, torch, rbl, synth, dev, args.max_tile_bytes, pre_bias=(opt == "pre_bias")))
        torch.cuda.synchronize()
        k2 = max(5, K // 2)
        next_info, _, _, _ = measure_layers(torch, rbl, extra, k2, W, s_main, s_aux)
        if "ffn_up" in next_info and "ffn_down" in layer_info:
            next_info["mlp_chain_fc1_swiglu_fc2_ms"] = round(next_info["ffn_up"]["ms"] + layer_info["ffn_down"]["ms"], 4)
        del extra

    w4_info = None
    w4_names = [n.strip() for n in args.w4a8.split(",") if n.strip()]
    if w4_names:
        print(f"bench: W4A8 variant on {w4_names}", file=sys.stderr, flush=True)
        w4_info = w4a8_layers(torch, rbl, synth, dev, w4_names, s_main, n=max(5, K // 2))
        w4_info["value_ms_per_layer"] = round(sum(v["layer_ms"] for v in w4_info.values()) / len(w4_names), 4)

    w44_info = None
    w44_names = [n.strip() for n in args.w4a4.split(",") if n.strip()]
    if w44_names:
        print(f"bench: W4A4 variant on {w44_names}", file=sys.stderr, flush=True)
        w44_info = w4a4_layers(torch, rbl, synth, dev, w44_names, s_main, n=max(5, K // 2))
        w44_info["value_ms_per_layer"] = round(sum(v["layer_ms"] for v in w44_info.values()) / len(w44_names), 4)
        w44_info["e2m3_value_ms_per_layer"] = round(
            sum(w44_info[k]["e2m3"]["layer_ms"] for k in w44_names) / len(w44_names), 4)

    short_info = None
    rows_list = [int(v) for v in args.short_batches.split(",") if v.strip()]
    if rows_list:
        print(f"bench: short batches {rows_list} (decode-inside-GEMM)", file=sys.stderr, flush=True)
        short_info = short_batches(torch, rbl, synth, dev, s_main, rows_list)

    dom = layers[0]
    dom_info = layer_info[dom.name]
    if dom.fused:
        # a short batch: the decode-inside-GEMM kernel, bound by vector issue
        achieved = FUSED_VALU_PER_ELEM * dom.w.N * dom.w.K_pad / (dom_info["split"]["gemm_ms"] * 1e-3) / 1e12
        roofline = {
            "kernel": f"gemm_nvfp4_fused ({dom.name}: M={dom.w.M} N={dom.w.N} K_pad={dom.w.K_pad})",
            "bound": "alu", "achieved": round(achieved, 2), "peak": PEAK_VALU_TOPS, "unit": "Tops/s",
            "frac": round(achieved / PEAK_VALU_TOPS, 4), "traffic": None,
            "per_element_ops": FUSED_VALU_PER_ELEM,
        }
    else:
        # per launch: algorithmic ops of one chunk's GEMM over its mean launch duration
        # (events around each GEMM launch of the component mirror, on the main stream)
        launch_ops = dom.gemm_ops / dom.nchunks
        launch_ms = dom_info["split"]["gemm_ms"] / dom.nchunks
        achieved = launch_ops / (launch_ms * 1e-3) / 1e12
        launch_shape = (dom.w.M, dom.chunks[0][1], dom.w.K_pad)
        roofline = {
            "kernel": (f"gemm_s8_rowscale ({dom.name}: {dom.nchunks} launch(es) of M={launch_shape[0]} "
                       f"N={launch_shape[1]} K_pad={launch_shape[2]})"),
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOP/s",
            "frac": round(achieved / PEAK_INT8_TOPS, 4),
            "traffic": counter_traffic(launch_shape),
            "launch_ms": round(launch_ms, 4),
            "per_launch_ops": launch_ops,
        }
    result = {
        "metric": METRIC,
        "value": round(sum(v["ms"] for v in layer_info.values()) / len(layer_info), 4),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "; ".join(L.w.note for L in layers),
            "M": layers[0].w.M,
            "layers": names,
            "timed_call": "cr_linear_nvfp4 (one call per layer, events on the calling stream)",
            "inputs": "bf16 activations ~N(0,1) (QKV: 1% channels x20), NVFP4 weights from 0.02*N(0,1)",
            "weight_prep_stream": "second stream" if args.two_stream else "calling stream (serial staging)",
            "max_tile_bytes": args.max_tile_bytes or rbl.DEFAULT_MAX_TILE_BYTES,
        },
        "roofline": roofline,
        "layers": layer_info,
        "component_mirror_ms_per_step": round(mirror_step, 4),
        "bounded_staging": staging,
        "other_staging": other_staging,
        "configs": cfg_info,
        "next_shapes": next_info,
        "short_batches": short_info,
        "w4a8": w4_info,
        "w4a4": w44_info,
        "wall_ms_timed_region": round(wall_ms, 2),
        "copy_gbs": round(copy_gbs, 1),
        "gemm_source_sha256_16": gemm_source_hash(),
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(layers, args.cpu_sample_rows)
    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
