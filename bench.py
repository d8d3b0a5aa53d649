"""Benchmark of the block-scaled FP4 hot path on one MI355X.

One step = one full FP4 training pass of a linear layer at the up-projection shape
(8192 tokens, 4096 -> 14336): amax sampling on sample steps (per-operand D=50 caches),
quantize X (row view) and W, fprop Y = X W^T, stochastic-rounded dY in the row view and
dgrad dX = dY W, the wgrad views dY^T (T = 2048) and X^T (optionally H16-rotated) and
wgrad dW = dY^T X. Inputs are seeded synthetic tensors already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--fmt mxfp4|ue5m3|e4m3] [--hadamard 0|16|32]

Prints one JSON line. ``value`` = FP4 GEMM FLOPs of the step / step wall time (TFLOP/s).
``roofline`` is the GEMM kernel's achieved FLOP rate against the FP4 MFMA peak: the three
GEMMs of the step (fprop 8192x14336 K=4096, dgrad 8192x4096 K=14336, wgrad 14336x4096
K=8192) each do 2*8192*4096*14336 FLOP, and their launches are timed with HIP events on
the launch stream. ``traffic`` is the HBM bytes per GEMM launch from the FETCH_SIZE and
WRITE_SIZE counters, scaled by the counters' reading for a plain device copy of known
size; it is read from the profile summary under ``profiles/`` and is null when the GEMM
kernel sources changed since those counters were taken. ``quantizer`` is the row-view
activation quantizer's algorithmic GB/s against HBM peak; ``quantizer_rowcol`` the fused
ROW+COL quantizer's; ``step_quantizers`` the stochastic ROW+COL pass of dY and the weight
quantizer (TILE2D for UE5M3/E4M3); ``producer_fusion`` the fprop whose epilogue writes the
next layer's FP4 operand against fprop + a separate quantize; ``routes`` the same step in
the other scale formats (UE5M3 block 16 with 2D weights and D = 50 caches, E4M3, MXFP4),
each GEMM's fraction of the FP4 and the fp16/bf16 MFMA peaks; ``next_rows`` the
graph-timed fake-quant, decode, MXFP4->FP8 and tile-local quantizer kernels on the same
activation. ``cpu_baseline`` times the CPU oracle on bounded slices of the same workload
(all BLAS threads and one thread) and its quantizer on the full activation of every
workload (``--cpu-full``: every operand and view). ``--calib-copy-mib N`` runs one plain
N-MiB device copy before warm-up, the known-size reference for the byte counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

M_TOK, K_IN, N_OUT = 8192, 4096, 14336
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense FP4/FP6 MFMA
BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
METRIC = "FP4 GEMM TFLOPS + quantize GB/s at 8192x4096x14336, % of MI355X peak"
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "fp4_block_scaled_tensor_amd", "csrc")
GEMM_SOURCES = {"mxfp4": ["gemm_mx.hip", "gemm_common.hpp", "fp4_device.hpp"],
                "ue5m3": ["gemm_dec16.hip", "gemm_common.hpp", "fp4_device.hpp"],
                "e4m3": ["gemm_dec16.hip", "gemm_common.hpp", "fp4_device.hpp"]}
GEMM_KERNEL = {"mxfp4": "k_gemm_mx", "ue5m3": "k_gemm_dec16", "e4m3": "k_gemm_dec16"}
GEMM_KERNEL_PRE = "k_gemm_f16_w8"   # --predecode (UE5M3/E4M3 block 16)


def log(msg):
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--fmt", default="mxfp4", choices=["mxfp4", "ue5m3", "e4m3"])
    p.add_argument("--hadamard", type=int, default=0, choices=[0, 16, 32])
    p.add_argument("--separate", action="store_true",
                   help="quantize the ROW and COL views of X and dY with two calls instead of the fused one")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=384, help="output rows of the oracle GEMM sample")
    p.add_argument("--calib-copy-mib", type=int, default=0, help="one plain device copy of this size first")
    p.add_argument("--no-routes", action="store_true", help="skip the other scale formats' steps")
    p.add_argument("--predecode", action="store_true",
                   help="UE5M3/E4M3: decode each GEMM's operands once to fp16 and run the decode-once GEMM")
    p.add_argument("--cpu-full", action="store_true",
                   help="also time the oracle quantizer on the full tensors of every workload (minutes)")
    return p.parse_args()


def gemm_source_hash(fmt_name):
    h = hashlib.sha256()
    for f in GEMM_SOURCES[fmt_name]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(fmt_name, kernel=None):
    """HBM bytes per GEMM launch recorded in profiles/, if taken on the current kernel sources."""
    kernel = kernel or GEMM_KERNEL[fmt_name]
    path = os.path.join(ROOT, "profiles", f"{kernel}_{fmt_name}_8192x4096x14336_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha256_16") != gemm_source_hash(fmt_name):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class LinearStep:
    """Buffers and per-operand amax caches of one FP4 linear layer (fprop + dgrad + wgrad)."""

    def __init__(self, fp4, torch, X, W, dY, fmt_name, hadamard, fused=True, predecode=False):
        self.fp4, self.torch = fp4, torch
        self.fused = fused
        self.predecode = predecode and fmt_name != "mxfp4"
        self.buf16 = {}       # persistent fp16 decode buffers of the decode-once route
        self.evd = []         # around each pair of operand decodes
        self.X, self.W, self.dY = X, W, dY
        self.hn = hadamard
        self.fmt = {"mxfp4": fp4.E8M0, "ue5m3": fp4.UE5M3, "e4m3": fp4.E4M3}[fmt_name]
        self.block = 32 if self.fmt == fp4.E8M0 else 16
        D = 1 if self.fmt == fp4.E4M3 else 50          # E4M3 recipe: current scaling
        mk = lambda: fp4.AmaxCache(D)
        self.c_x, self.c_w, self.c_dy = mk(), mk(), mk()
        self.c_xh, self.c_dyh = (mk(), mk()) if hadamard else (self.c_x, self.c_dy)
        self.obs = torch.empty(1, dtype=torch.float32, device="cuda")
        dev = "cuda"
        self.Y = torch.empty((M_TOK, N_OUT), dtype=torch.float32, device=dev)
        self.dX = torch.empty((M_TOK, K_IN), dtype=torch.float32, device=dev)
        self.dW = torch.empty((N_OUT, K_IN), dtype=torch.float32, device=dev)
        self.ev = []          # (start, end) events around each GEMM launch
        self.evq = []         # around each activation row-view quantization

    def _timed(self, timed, fn, *a, **kw):
        if not timed:
            return fn(*a, **kw)
        e0, e1 = self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)
        e0.record()
        r = fn(*a, **kw)
        e1.record()
        self.ev.append((e0, e1))
        return r

    def _gemm(self, timed, name, a, b, out, hadamard_n=0):
        """One GEMM of the step; with predecode, both operands are first decoded once into fp16
        (fp4_decode_f16, timed apart) and the decode-once kernel (fp4_gemm_f16) runs."""
        fp4, torch = self.fp4, self.torch
        if not self.predecode:
            if name == "wgrad":
                return self._timed(timed, fp4.gemm_wgrad, a, b, hadamard_n=hadamard_n, out=out)
            return self._timed(timed, getattr(fp4, "gemm_" + name), a, b, out=out)
        bufs = []
        for tag, op in (("a", a), ("b", b)):
            key = (name, tag)
            if key not in self.buf16:
                self.buf16[key] = torch.empty((op.rows, op.k), dtype=torch.float16, device="cuda")
            bufs.append(self.buf16[key])
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        fp4.decode_f16(a, out=bufs[0])
        fp4.decode_f16(b, out=bufs[1])
        if timed:
            e1.record()
            self.evd.append((e0, e1))
        return self._timed(timed, fp4.gemm_f16, a, b, a16=bufs[0], b16=bufs[1], hadamard_n=hadamard_n, out=out)

    def _sample(self, cache, x, step, hn=0):
        if self.fmt == self.fp4.E8M0:
            return
        if cache.needs_sample(step):
            self.fp4.tensor_amax(x, hn, out=self.obs)
            cache.update(step, self.obs)

    def run(self, step, timed=False):
        fp4, torch = self.fp4, self.torch
        E8 = self.fmt == fp4.E8M0
        B = self.block
        # forward: X is quantized once for fprop (ROW) and, in the same pass when fused, for
        # wgrad (COL, saved for the backward)
        self._sample(self.c_x, self.X, step)
        self._sample(self.c_xh, self.X, step, self.hn)
        self._sample(self.c_w, self.W, step)
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        if self.fused:
            qx, qxt = fp4.quantize_rowcol(self.X, self.fmt, B, amax_row=self.c_x.amax, amax_col=self.c_xh.amax,
                                          T_row=448, T_col=448, hadamard_n=self.hn)
        else:
            qx = fp4.quantize(self.X, self.fmt, B, fp4.ROW, amax=self.c_x.amax, T=448)
        if timed:
            e1.record()
            self.evq.append((e0, e1))
        if E8:
            if self.fused:   # W for fprop and W^T (blocks along out-features) for dgrad, one read
                qw, qwt = fp4.quantize_rowcol(self.W, self.fmt, B)
            else:
                qw = fp4.quantize(self.W, self.fmt, B, fp4.ROW)
                qwt = fp4.quantize(self.W, self.fmt, B, fp4.COL)
        else:
            qw, qwt = fp4.quantize(self.W, self.fmt, 16, fp4.TILE2D, amax=self.c_w.amax, T=448)
        self._gemm(timed, "fprop", qx, qw, self.Y)
        # backward: dY for dgrad (ROW, T = 448) and wgrad (COL, T = 2048, optional Hadamard),
        # both with stochastic rounding
        self._sample(self.c_dy, self.dY, step)
        self._sample(self.c_dyh, self.dY, step, self.hn)
        if self.fused:
            qdy, qdyt = fp4.quantize_rowcol(self.dY, self.fmt, B, amax_row=self.c_dy.amax, amax_col=self.c_dyh.amax,
                                            T_row=448, T_col=2048, stochastic_row=True, stochastic_col=True,
                                            seed_row=42, offset_row=step * 8 + 0, seed_col=42,
                                            offset_col=step * 8 + 1, hadamard_n=self.hn)
        else:
            qdy = fp4.quantize(self.dY, self.fmt, B, fp4.ROW, amax=self.c_dy.amax, T=448, stochastic=True, seed=42,
                               offset=step * 8 + 0)
            qdyt = fp4.quantize(self.dY, self.fmt, B, fp4.COL, amax=self.c_dyh.amax, T=2048, stochastic=True,
                                seed=42, offset=step * 8 + 1, hadamard_n=self.hn)
        self._gemm(timed, "dgrad", qdy, qwt, self.dX)
        if not self.fused:
            qxt = fp4.quantize(self.X, self.fmt, B, fp4.COL, amax=self.c_xh.amax, T=448, hadamard_n=self.hn)
        self._gemm(timed, "wgrad", qdyt, qxt, self.dW, hadamard_n=self.hn)


# Graph-timed kernels read their input from one of NROT identical copies in turn, so the
# inputs of back-to-back calls (NROT x 67 MB for the 8192x4096 activation) exceed the 256 MB
# last-level cache and every call reads HBM.
NROT = 8


def graph_time_ms(torch, fn, check, reps=20):
    """Average GPU time of fn(i) from one replay of a captured HIP graph of reps back-to-back
    calls (no host launch gaps); call k uses input copy k % NROT. check(out) compares a
    replay's output with an eager call's; returns (ms, ok)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    outs = []
    with torch.cuda.graph(g):
        for k in range(reps):
            outs.append(fn(k % NROT))
    g.replay()
    torch.cuda.synchronize()
    ok = check(outs[-1])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(3):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / reps)
    ok = ok and check(outs[-1])
    del g
    return best, ok


def next_rows(torch, fp4, Xrot, step_obj, args):
    """Graph-timed kernels of the rows built past the training step, on the same 8192x4096
    activation: inference fake quantization (bf16 out) and operand decode, MXFP4 -> FP8
    (transposed, the backward form), tile-local quantization (E4M3, 16- and 128-row stripes). Each
    entry: algorithmic bytes per element, average ms, GB/s and fraction of HBM peak."""
    n = M_TOK * K_IN
    fmt, B = step_obj.fmt, step_obj.block
    amax = None if fmt == fp4.E8M0 else step_obj.c_x.amax
    q_row = [fp4.quantize(x, fmt, B, fp4.ROW, amax=amax, T=448) for x in Xrot]
    q_mx = [fp4.quantize(x, fp4.E8M0, 32, fp4.ROW) for x in Xrot]
    torch.cuda.synchronize()
    cases = {
        "fake_quant": ("k_fake_quant (bf16 in, bf16 out)", 4.0,
                       lambda i: fp4.fake_quant(Xrot[i], fmt, B, amax=amax, T=448, out_dtype=torch.bfloat16),
                       lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16))),
        "dequantize": ("k_dequant (bf16 out)", 0.5 + 1.0 / B + 2.0,
                       lambda i: fp4.dequantize(q_row[i], out_dtype=torch.bfloat16),
                       lambda a, b: torch.equal(a.view(torch.int16), b.view(torch.int16))),
        "mxfp4_to_fp8": ("k_mx_to_fp8 (transposed out)", 0.5 + 1.0 / 32 + 1.0 + 1.0 / 128,
                         lambda i: fp4.mxfp4_to_fp8(q_mx[i], transpose=True),
                         lambda a, b: torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])),
        "quantize_local": ("k_quant_row_local (E4M3, 16-row stripes)", 2.0 + 0.5 + 1.0 / 16,
                           lambda i: fp4.quantize_local(Xrot[i], fp4.E4M3, 16, stripe=16),
                           lambda a, b: torch.equal(a.q, b.q) and torch.equal(a.s, b.s) and torch.equal(a.g, b.g)),
        "quantize_local_s128": ("k_stripe_amax + k_quant_row (E4M3, 128-row stripes, two-pass)", 2.0 + 0.5 + 1.0 / 16,
                                lambda i: fp4.quantize_local(Xrot[i], fp4.E4M3, 16, stripe=128),
                                lambda a, b: torch.equal(a.q, b.q) and torch.equal(a.s, b.s) and torch.equal(a.g, b.g)),
    }
    out = {}
    for name, (kernel, bpe, fn, same) in cases.items():
        ref = fn(0)
        torch.cuda.synchronize()
        ms, ok = graph_time_ms(torch, fn, lambda o: same(o, ref))
        gbs = n * bpe / (ms * 1e-3) / 1e9
        out[name] = {"kernel": kernel, "bytes_per_elem": round(bpe, 6), "avg_ms": round(ms, 4),
                     "achieved": round(gbs, 1), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "replay_matches_eager": ok}
    return out


def time_step(torch, step_obj, warmup, steps, first_step=0):
    """(ms per step, average ms per GEMM launch) of `steps` timed steps after `warmup` untimed."""
    for s in range(first_step, first_step + warmup):
        step_obj.run(s)
    torch.cuda.synchronize()
    step_obj.ev.clear()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(first_step + warmup, first_step + warmup + steps):
        step_obj.run(s, timed=True)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps, float(np.mean([a.elapsed_time(b) for a, b in step_obj.ev]))


def routes(torch, fp4, Xd, Wd, dYd, args, skip):
    """The same training step in the other scale formats: UE5M3 block 16 with 2D weights and
    D = 50 caches (the main recipe), E4M3 block 16 with D = 1 (current scaling), each with the
    per-workgroup decode and with each GEMM's operands decoded once to fp16 (the decode passes
    inside the step and timed apart), and MXFP4. Each: ms per step, the GEMM kernel's average
    launch, its TFLOP/s and fractions of the FP4 and the fp16/bf16 MFMA peaks (the decoded
    routes' true ceiling)."""
    out = {}
    flop_gemm = 2.0 * M_TOK * N_OUT * K_IN
    for route in ("ue5m3", "ue5m3_decode_once", "e4m3", "e4m3_decode_once", "mxfp4"):
        name = route.split("_")[0]
        pre = route.endswith("decode_once")
        if name == skip and pre == args.predecode:     # the headline step itself
            continue
        st = LinearStep(fp4, torch, Xd, Wd, dYd, name, args.hadamard, predecode=pre)
        ms_step, gemm_ms = time_step(torch, st, 3, 10)
        tf = flop_gemm / (gemm_ms * 1e-3) / 1e12
        out[route] = {"ms_per_step": round(ms_step, 4), "step_TFLOPs": round(3 * flop_gemm / (ms_step * 1e-3) / 1e12, 1),
                     "gemm_kernel": GEMM_KERNEL_PRE if pre else GEMM_KERNEL[name], "gemm_avg_ms": round(gemm_ms, 4),
                     "decode_pair_avg_ms": round(float(np.mean([a.elapsed_time(b) for a, b in st.evd])), 4) if pre
                     else None,
                     "gemm_TFLOPs": round(tf, 1), "frac_of_fp4_peak": round(tf / FP4_PEAK_TFLOPS, 4),
                     "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                     "recipe": {"ue5m3": "UE5M3 block 16, W 2D 16x16, D=50 caches, SR dY, T=2048 wgrad dY",
                                "e4m3": "E4M3 block 16 + fp32 tensor scale, W 2D, D=1 (current), SR dY",
                                "mxfp4": "E8M0 block 32, no tensor scale, SR dY"}[name]
                               + ("; each GEMM's operands decoded once to fp16 (inside the step)" if pre else "")}
        del st
        torch.cuda.empty_cache()
    return out


def step_kernels(torch, fp4, Xd, Wd, dYd, step_obj):
    """Graph-timed quantizers of the step not covered above: the stochastic fused ROW+COL pass of
    dY (8192 x 14336, both views SR, T = 2048 for the COL view) and the weight quantizer
    (TILE2D for UE5M3/E4M3: 14336 x 4096 -> forward and transposed payload plus the shared
    16x16 grid; the fused ROW+COL pass for MXFP4)."""
    fmt, B = step_obj.fmt, step_obj.block
    E8 = fmt == fp4.E8M0
    out = {}
    dyrot = [dYd] + [dYd.clone() for _ in range(2)]          # 3 x 235 MB: past the last-level cache
    ady = None if E8 else step_obj.c_dy.amax
    fn = lambda i: fp4.quantize_rowcol(dyrot[i % 3], fmt, B, amax_row=ady, amax_col=ady, T_row=448, T_col=2048,
                                       stochastic_row=True, stochastic_col=True, seed_row=42, offset_row=8,
                                       seed_col=42, offset_col=9)
    ref = fn(0)
    torch.cuda.synchronize()
    ms, ok = graph_time_ms(torch, fn, lambda o: all(torch.equal(a.q, b.q) and torch.equal(a.s, b.s)
                                                   for a, b in zip(o, ref)))
    n = M_TOK * N_OUT
    bpe = 2 + 2 * (0.5 + 1.0 / B)
    gbs = n * bpe / (ms * 1e-3) / 1e9
    out["sr_rowcol_dY"] = {"kernel": "k_quant_rowcol (dY 8192x14336 bf16, SR both views)", "bytes_per_elem": bpe,
                           "avg_ms": round(ms, 4), "achieved": round(gbs, 1), "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4), "replay_matches_eager": ok,
                           "bound": "VALU (Philox-4x32-10 draws and the stochastic E2M1 decision)"}
    del dyrot
    wrot = [Wd] + [Wd.clone() for _ in range(3)]              # 4 x 117 MB
    if E8:
        fn = lambda i: fp4.quantize_rowcol(wrot[i % 4], fmt, B)
        kern, wbpe = "k_quant_rowcol (W 14336x4096, ROW + COL)", 2 + 2 * (0.5 + 1.0 / 32)
    else:
        aw = step_obj.c_w.amax
        fn = lambda i: fp4.quantize(wrot[i % 4], fmt, 16, fp4.TILE2D, amax=aw, T=448)
        kern, wbpe = "k_quant_2d (W 14336x4096, TILE2D)", 2 + 0.5 + 0.5 + 1.0 / 256
    ref = fn(0)
    torch.cuda.synchronize()
    ms, ok = graph_time_ms(torch, fn, lambda o: all(torch.equal(a.q, b.q) and torch.equal(a.s, b.s)
                                                   for a, b in zip(o, ref)))
    n = N_OUT * K_IN
    gbs = n * wbpe / (ms * 1e-3) / 1e9
    out["weight"] = {"kernel": kern, "bytes_per_elem": round(wbpe, 6), "avg_ms": round(ms, 4),
                     "achieved": round(gbs, 1), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "replay_matches_eager": ok}
    del wrot
    # the COL view alone (the unfused form of the wgrad operand): X^T of the activation
    xrot = [Xd] + [Xd.clone() for _ in range(NROT - 1)]
    ax = None if E8 else step_obj.c_x.amax
    fn = lambda i: fp4.quantize(xrot[i], fmt, B, fp4.COL, amax=ax, T=448)
    ref = fn(0)
    torch.cuda.synchronize()
    ms, ok = graph_time_ms(torch, fn, lambda o: torch.equal(o.q, ref.q) and torch.equal(o.s, ref.s))
    cbpe = 2 + 0.5 + 1.0 / B
    gbs = M_TOK * K_IN * cbpe / (ms * 1e-3) / 1e9
    out["col_view_X"] = {"kernel": "k_quant_col (X 8192x4096 -> X^T operand)", "bytes_per_elem": round(cbpe, 6),
                         "avg_ms": round(ms, 4), "achieved": round(gbs, 1), "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "replay_matches_eager": ok}
    return out


def producer_fusion(torch, fp4, step_obj):
    """The fprop whose epilogue writes Y as the next layer's FP4 operand (fp4_gemm_fprop_q, no
    float32 Y) against the float32 fprop followed by a separate ROW quantization of Y: bytes
    written per output element and the time of each route (events, 10 launches each)."""
    fmt, B = step_obj.fmt, step_obj.block
    E8 = fmt == fp4.E8M0
    amx = None if E8 else step_obj.c_x.amax
    qx = fp4.quantize(step_obj.X, fmt, B, fp4.ROW, amax=amx, T=448)
    if E8:
        qw = fp4.quantize(step_obj.W, fmt, B, fp4.ROW)
    else:
        qw, _ = fp4.quantize(step_obj.W, fmt, 16, fp4.TILE2D, amax=step_obj.c_w.amax, T=448)
    a_out = torch.tensor([4.0], dtype=torch.float32, device="cuda")
    Y = torch.empty((M_TOK, N_OUT), dtype=torch.float32, device="cuda")

    def fused():
        return fp4.gemm_fprop_q(qx, qw, fmt, B, amax=None if E8 else a_out, T=448)

    def separate():
        fp4.gemm_fprop(qx, qw, out=Y)
        return fp4.quantize(Y, fmt, B, fp4.ROW, amax=None if E8 else a_out, T=448)

    res = {}
    for name, fn in (("fused", fused), ("separate", separate)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / 10
    fq = fused()[0]
    sq = separate()
    torch.cuda.synchronize()
    same = bool(torch.equal(fq.q, sq.q) and torch.equal(fq.s, sq.s))
    return {"kernel": GEMM_KERNEL[{fp4.E8M0: "mxfp4", fp4.UE5M3: "ue5m3", fp4.E4M3: "e4m3"}[fmt]] + " with the "
                      "output quantized in its epilogue (fp4_gemm_fprop_q)",
            "bytes_written_per_output": round(0.5 + 1.0 / B, 6), "bytes_written_per_output_f32": 4.0,
            "separate_bytes_per_output": round(4.0 + 4.0 + 0.5 + 1.0 / B, 6),
            "fused_ms": round(res["fused"], 4), "fprop_then_quantize_ms": round(res["separate"], 4),
            "identical_to_separate": same}


def bf16_device(torch, synth, x):
    bits = synth.f32_to_bf16_bits(x)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def cpu_model() -> str:
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_gemm_seconds(oracle, OF, fmt, block, Xs, W, rows, amax_x):
    qx = oracle.quantize_1d(Xs[:rows], fmt, block, amax=amax_x, T=448)
    if fmt == OF.E8M0:
        qw = oracle.quantize_1d(W, fmt, block)
        b, sb = oracle.operand_from_quant(qw)
    else:
        qw = oracle.quantize_2d(W, fmt, amax=float(np.max(np.abs(W))), T=448)
        b, sb = oracle.operand_from_quant(qw, "2d")
    a, sa = oracle.operand_from_quant(qx)
    t1 = time.perf_counter()
    oracle.gemm_model(a, sa, b, sb, block, alpha=oracle.output_scale(qx.g, qw.g))
    return time.perf_counter() - t1


def oracle_full_tensors(oracle, OF, synth, every_view):
    """The oracle quantizer on full tensors of each workload: the tiny 256x256 pair, the 2048^3
    format sweep (all three formats), the up-projection, the down-projection backward and one
    step of the 8B layer set. By default the activation (or dY) of each, ROW view; with
    every_view every operand in each view its GEMMs read (ROW, COL with T = 2048 and SR for dY,
    2D for UE5M3/E4M3 weights). Returns {workload: {elements, seconds, GBps}}."""
    U, E4, E8 = OF.UE5M3, OF.E4M3, OF.E8M0
    res = {}

    def q(name, x, fmt, view="row", sr=False, T=448.0, src_bytes=2):
        B = 32 if fmt == E8 else 16
        A = None if fmt == E8 else float(np.max(np.abs(x)))
        t0 = time.perf_counter()
        if view == "2d":
            oracle.quantize_2d(x, fmt, amax=A, T=T)
            out_b = 2 * 0.5 + 1.0 / 256
        else:
            xv = np.ascontiguousarray(x.T) if view == "col" else x
            oracle.quantize_1d(xv, fmt, B, amax=A, T=T, rounding="sr" if sr else "rne", seed=42, offset=0)
            out_b = 0.5 + 1.0 / B
        dt = time.perf_counter() - t0
        log(f"oracle quantizer, {name}: {x.shape[0]}x{x.shape[1]} {view} {dt:.2f} s")
        r = res.setdefault(name, {"elements": 0, "seconds": 0.0, "bytes": 0.0})
        r["elements"] += x.size
        r["seconds"] += dt
        r["bytes"] += x.size * (src_bytes + out_b)

    c1 = synth.make_config(1)
    q("tiny 256x256 fp32 (UE5M3)", c1["X"].values, U, src_bytes=4)
    if every_view:
        q("tiny 256x256 fp32 (UE5M3)", c1["W"].values, U, src_bytes=4)
    c2 = synth.make_config(2)
    for f in (U, E4, E8):
        q("format sweep 2048^3 bf16 (3 formats)", c2["X"].values, f)
        if every_view:
            q("format sweep 2048^3 bf16 (3 formats)", c2["W"].values, f)
    del c2
    bf16 = lambda x: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    key = "up-projection 8192x4096 -> 14336"
    if every_view:
        c3 = synth.make_config(3)
        q(key, c3["X"].values, U)
        q(key, c3["W"].values, U, "2d")
        del c3
    else:                               # the same seeded activation, without drawing W
        X, _ = synth.scale_channels(synth.student_t((M_TOK, K_IN), 3.0, 301), 4, 100.0, 302)
        q(key, bf16(X), U)
        del X
    key = "down-projection backward 8192 tok, 4096 x 21504"
    if every_view:
        c4 = synth.make_config(4)
        q(key, c4["dY"].values, U, sr=True)
        q(key, c4["dY"].values, U, "col", sr=True, T=2048.0)
        q(key, c4["W"].values, U, "2d")
        q(key, c4["X"].values, U, "col")
        del c4
    else:
        q(key, bf16(synth.normal((M_TOK, 4096), 1e-3, 401)), U, sr=True)
    for layer, (lname, in_f, out_f) in enumerate(synth.LINEARS_8B):
        if not every_view and layer > 0:
            break
        base = synth.layer_base(layer, synth.C5_TOKENS, in_f, out_f)
        key = "8B layer set, step 0 at 8192 tokens" + ("" if every_view else " (qkv X)")
        toks = synth.C5_TOKENS
        X = synth.drift_np(base["X"], synth.step_perm(layer, "X", 0, toks), synth.step_amp(0)).values
        q(key, X, U)
        if every_view:
            dY = synth.drift_np(base["dY"], synth.step_perm(layer, "dY", 0, toks), synth.step_amp(0)).values
            q(key, X, U, "col")
            q(key, dY, U, sr=True)
            q(key, dY, U, "col", sr=True, T=2048.0 if lname == "down" else 448.0)
            q(key, synth.layer_weight(layer, out_f, in_f).values, U, "2d")
            del dY
        del base, X
    for r in res.values():
        r["GBps"] = round(r["bytes"] / r["seconds"] / 1e9, 6)
        r["seconds"] = round(r["seconds"], 3)
        del r["bytes"]
    return res


def oracle_gemm_full(oracle, OF, synth, every_format):
    """The oracle's group-model GEMM over whole workloads small enough to run in full: the tiny
    256x256x256 pair (UE5M3, 1D) and the 2048^3 format sweep (UE5M3; with every_format also
    E4M3 and MXFP4). Quantization untimed. Returns {workload: {seconds, GFLOPs}}."""
    res = {}

    def one(name, X, W, fmt):
        B = 32 if fmt == OF.E8M0 else 16
        ax = None if fmt == OF.E8M0 else float(np.max(np.abs(X)))
        aw = None if fmt == OF.E8M0 else float(np.max(np.abs(W)))
        qx = oracle.quantize_1d(X, fmt, B, amax=ax, T=448)
        qw = oracle.quantize_1d(W, fmt, B, amax=aw, T=448)
        a, sa = oracle.operand_from_quant(qx)
        b, sb = oracle.operand_from_quant(qw)
        t0 = time.perf_counter()
        oracle.gemm_model(a, sa, b, sb, B, alpha=oracle.output_scale(qx.g, qw.g))
        dt = time.perf_counter() - t0
        fl = 2.0 * X.shape[0] * W.shape[0] * X.shape[1]
        res[name] = {"seconds": round(dt, 3), "GFLOPs": round(fl / dt / 1e9, 4)}
        log(f"oracle GEMM, {name}: {dt:.2f} s")

    c1 = synth.make_config(1)
    one("tiny 256x256x256 (UE5M3)", c1["X"].values, c1["W"].values, OF.UE5M3)
    c2 = synth.make_config(2)
    for fmt, nm in ((OF.UE5M3, "UE5M3"), (OF.E4M3, "E4M3"), (OF.E8M0, "MXFP4")):
        if fmt != OF.UE5M3 and not every_format:
            continue
        one(f"format sweep 2048^3 ({nm})", c2["X"].values, c2["W"].values, fmt)
    return res


def cpu_baseline(args, fmt_name, synth):
    """The oracle as it stands, on the host, on bounded slices of the same workload:
    the group-model GEMM for args.cpu_rows output rows across all 14336 columns (W quantized
    in full, untimed) with every BLAS thread (and the full up-projection's time extrapolated
    linearly in M from it), the same GEMM for 32 rows on one thread, the GEMM over the tiny and
    format-sweep workloads in full, and the oracle quantizer on the full activation tensor of
    every workload; the speed-up of the GPU kernels over the oracle."""
    import oracle
    from oracle import formats as OF
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    fmt = {"mxfp4": OF.E8M0, "ue5m3": OF.UE5M3, "e4m3": OF.E4M3}[fmt_name]
    block = 32 if fmt == OF.E8M0 else 16
    rows, rows1 = args.cpu_rows, 32
    Xs = synth.student_t((max(rows, 1024), K_IN), 3.0, 301)
    Xs, _ = synth.scale_channels(Xs, 4, 100.0, 302)
    W = synth.normal((N_OUT, K_IN), 0.02, 303)
    amax_x = float(np.max(np.abs(Xs)))
    tg = oracle_gemm_seconds(oracle, OF, fmt, block, Xs, W, rows, amax_x)
    with threadpool_limits(1):
        tg1 = oracle_gemm_seconds(oracle, OF, fmt, block, Xs, W, rows1, amax_x)
        t0 = time.perf_counter()
        oracle.quantize_1d(Xs[:1024], fmt, block, amax=amax_x, T=448)
        tq1 = time.perf_counter() - t0
    del Xs, W
    full = oracle_full_tensors(oracle, OF, synth, args.cpu_full)
    gemm_full = oracle_gemm_full(oracle, OF, synth, args.cpu_full)
    flops_row = 2.0 * N_OUT * K_IN
    qbytes1 = 1024 * K_IN * (2 + 0.5 + 1.0 / block)
    up = full["up-projection 8192x4096 -> 14336"]
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": round(rows * flops_row / tg / 1e12, 8), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"group-model GEMM of {rows} output rows x {N_OUT} cols, K={K_IN} ({fmt_name}): {tg:.1f} s "
                      f"on {threads} BLAS threads",
            "one_thread": {"value": round(rows1 * flops_row / tg1 / 1e12, 8), "unit": "TFLOP/s",
                           "sample": f"the same GEMM for {rows1} rows: {tg1:.1f} s; row-view quantizer on "
                                     f"1024x{K_IN}: {tq1:.2f} s",
                           "quantizer_GBps": round(qbytes1 / tq1 / 1e9, 6)},
            "quantizer_GBps": up["GBps"],
            "gemm_full_workloads": gemm_full,
            "up_projection_gemm_estimate_s": round(tg * M_TOK / rows, 1),
            "quantizer_full_tensors": full,
            "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": cpu_model(),
            "note": "the oracle quantizer is numpy elementwise code: one thread whatever the BLAS pool"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the FP4 hot path here runs on a single GPU; "
              "--gpus above 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import fp4_block_scaled_tensor_amd as fp4
    fp4.library()                     # fails loudly if the HIP library is missing
    torch.manual_seed(0)
    # synthetic inputs: the up-projection activation (Student-t nu=3, 4 outlier channels x100),
    # weight N(0, 0.02), upstream gradient N(0, 1e-3)
    X = synth.student_t((M_TOK, K_IN), 3.0, 301)
    X, _ = synth.scale_channels(X, 4, 100.0, 302)
    Xd = bf16_device(torch, synth, X)
    Wd = bf16_device(torch, synth, synth.normal((N_OUT, K_IN), 0.02, 303))
    dYd = bf16_device(torch, synth, synth.normal((M_TOK, N_OUT), 1e-3, 304))
    del X
    step_obj = LinearStep(fp4, torch, Xd, Wd, dYd, args.fmt, args.hadamard, fused=not args.separate,
                          predecode=args.predecode)
    if args.calib_copy_mib > 0:
        # known-size reference for the HBM byte counters: one plain copy of N MiB
        src = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for s in range(args.warmup):
        step_obj.run(s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(args.warmup, args.warmup + args.steps):
        step_obj.run(s, timed=True)
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps
    gemm_ms = float(np.mean([a.elapsed_time(b) for a, b in step_obj.ev]))
    quant_ms_step = float(np.mean([a.elapsed_time(b) for a, b in step_obj.evq]))
    # the activation row-view quantizer alone, launch gaps excluded (graph replay)
    qargs = dict(amax=step_obj.c_x.amax, T=448) if step_obj.fmt != fp4.E8M0 else {}
    Xrot = [Xd] + [Xd.clone() for _ in range(NROT - 1)]
    qfn = lambda i: fp4.quantize(Xrot[i], step_obj.fmt, step_obj.block, fp4.ROW, **qargs)
    ref_q = qfn(0)
    torch.cuda.synchronize()
    same = lambda o: bool(torch.equal(o.q, ref_q.q) and torch.equal(o.s, ref_q.s))
    quant_ms, quant_ok = graph_time_ms(torch, qfn, same)
    if not quant_ok and args.separate:
        quant_ms = quant_ms_step
    # the fused ROW + COL activation quantizer (X for fprop and X^T for wgrad from one read)
    cargs = dict(amax_row=step_obj.c_x.amax, amax_col=step_obj.c_xh.amax) if step_obj.fmt != fp4.E8M0 else {}
    rcfn = lambda i: fp4.quantize_rowcol(Xrot[i], step_obj.fmt, step_obj.block, hadamard_n=args.hadamard, **cargs)
    ref_rc = rcfn(0)
    torch.cuda.synchronize()
    same_rc = lambda o: all(bool(torch.equal(a.q, b.q) and torch.equal(a.s, b.s)) for a, b in zip(o, ref_rc))
    rc_ms, rc_ok = graph_time_ms(torch, rcfn, same_rc)
    rc_bpe = 2 + 2 * (0.5 + 1.0 / step_obj.block)
    rc_gbs = M_TOK * K_IN * rc_bpe / (rc_ms * 1e-3) / 1e9
    log(f"step {ms_step:.3f} ms, GEMM {gemm_ms:.4f} ms; graph-timed quantizers")
    extra = next_rows(torch, fp4, Xrot, step_obj, args)
    log("producer fusion")
    fusion = producer_fusion(torch, fp4, step_obj)
    # measured HBM reference on the same rotated inputs: a plain device copy of the activation
    # (2 B/elem read + 2 written)
    cp_ms, _ = graph_time_ms(torch, lambda i: Xrot[i].clone(), lambda o: True)
    hbm_ref = {"copy_GBps": round(M_TOK * K_IN * 4 / (cp_ms * 1e-3) / 1e9, 1),
               "kernel": "device copy of the 8192x4096 bf16 activation (torch clone)",
               "timing": f"graph replay of 20 calls, inputs rotated over {NROT} copies"}
    del Xrot
    torch.cuda.empty_cache()
    log("step quantizers")
    kernels = step_kernels(torch, fp4, Xd, Wd, dYd, step_obj)
    log("other scale formats")
    other = {} if args.no_routes else routes(torch, fp4, Xd, Wd, dYd, args, args.fmt)
    flop_gemm = 2.0 * M_TOK * N_OUT * K_IN
    step_flops = 3 * flop_gemm
    gemm_kernel = GEMM_KERNEL_PRE if step_obj.predecode else GEMM_KERNEL[args.fmt]
    value = step_flops / (ms_step * 1e-3) / 1e12
    achieved = flop_gemm / (gemm_ms * 1e-3) / 1e12
    bpe = 2 + 0.5 + 1.0 / step_obj.block
    q_gbs = M_TOK * K_IN * bpe / (quant_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4-e2m1 (" + args.fmt + " scales), fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"FP4 linear training step 8192 tok x 4096 -> 14336 ({args.fmt}, H{args.hadamard})",
                   "tokens": M_TOK, "in_features": K_IN, "out_features": N_OUT, "gemms_per_step": 3,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": FP4_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / FP4_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profile(args.fmt, gemm_kernel),
                     "kernel": gemm_kernel + " (fprop, dgrad and wgrad launches, 2*8192*4096*14336 FLOP each)",
                     "avg_ms": round(gemm_ms, 4), "source_sha256_16": gemm_source_hash(args.fmt),
                     "frac_of_bf16_peak": None if args.fmt == "mxfp4" else round(achieved / BF16_PEAK_TFLOPS, 4)},
        "quantizer": {"kernel": "k_quant_row (activation 8192x4096 bf16)", "achieved": round(q_gbs, 1),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(q_gbs / HBM_PEAK_GBS, 4),
                      "bytes_per_elem": bpe, "avg_ms": round(quant_ms, 4),
                      "timing": f"graph replay of 20 calls, inputs rotated over {NROT} copies" if quant_ok else
                                ("events in the step" if args.separate else "graph replay check failed"),
                      "in_step_avg_ms": round(quant_ms_step, 4) if args.separate else None},
        "quantizer_rowcol": {"kernel": f"k_quant_rowcol (activation 8192x4096 bf16, COL view H{args.hadamard})",
                             "achieved": round(rc_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(rc_gbs / HBM_PEAK_GBS, 4), "bytes_per_elem": rc_bpe,
                             "avg_ms": round(rc_ms, 4), "replay_matches_eager": rc_ok,
                             "in_step_avg_ms": None if args.separate else round(quant_ms_step, 4)},
        "step_quantizers": kernels,
        "producer_fusion": fusion,
        "routes": other,
        "next_rows": extra,
        "hbm_reference": hbm_ref,
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        log("oracle on the host")
        out["cpu_baseline"] = cpu_baseline(args, args.fmt, synth)
        cb = out["cpu_baseline"]
        cb["speedup"] = {"gemm": round(achieved / cb["value"], 1),
                         "quantizer": round(q_gbs / cb["quantizer_GBps"], 1)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
