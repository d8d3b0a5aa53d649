"""Writes the expected values of the 8B layer set at seq 8192 (tests/test_gpu_layer_set_8192.py).

Every stored value comes from the oracle (and the seeded inputs of synth); nothing here runs
or reads the HIP library. Run from the repository root:

    python tests/golden/make_c5_golden.py [--workers 6]

It takes about ten minutes on 8 cores and writes
  tests/golden/c5_layer_set.json    digests of every quantized byte at the checked steps, the
                                    amax caches of every step, health counts of the stress run
  tests/golden/c5_gemm_samples.npz  sampled output blocks of the three GEMMs at the checked steps

Recipe ("UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", approach: UE5M3 block
16, T = 448, delayed amax caches with D = 50 per operand, 2D 16x16 weight scales, stochastic
rounding for dY only, T = 2048 for the weight-gradient dY operand of the down projection;
"技術概要：MXFP4 による大規模言語モデルの事前学習", method: H16 on the weight-gradient
operands, run with and without it):
  - four linears of one 8B layer (qkv 4096->6144, o 4096->4096, gate+up 4096->28672,
    down 14336->4096) at 8192 tokens over 100 steps; inputs from synth (layer_base,
    step_perm, step_amp with drift 1.02, drift_np); W fixed per layer;
  - one amax cache per (operand, rotation): x, x16, dy, dy16, w;
  - views per step: X ROW, X COL (H0, H16), dY ROW (SR, counter offset 8 step), dY COL (SR,
    H0 offset 8 step + 1, H16 offset 8 step + 2), W TILE2D;
  - stress: the o projection with drift 1.12 (beyond the 137x headroom at T = 448 after step 43,
    the 30x headroom at T = 2048 after about step 30), health counts of X ROW (T = 448),
    dY ROW (T = 448) and dY COL (T = 2048) at every step.
Large views are quantized in row (or feature) chunks with the oracle's own row offset, and
their digests are taken over the chunks in order, which equals the digest of the whole array.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
os.environ.setdefault("OMP_NUM_THREADS", "1")
os.environ.setdefault("OPENBLAS_NUM_THREADS", "1")

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402
from oracle import formats as OF  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
JSON_OUT = os.path.join(HERE, "c5_layer_set.json")
NPZ_OUT = os.path.join(HERE, "c5_gemm_samples.npz")

U = OF.UE5M3
B = 16
D = 50
SEED = 42
T_X = 448.0
T_DY_ROW = 448.0
CHUNK = 1024
STRESS_LAYER = 1
STRESS_DRIFT = 1.12
STRESS_HASH_STEPS = {"x_row": (43, 44), "dy_col": (30, 31)}


def t_dy_col(layer: int) -> float:
    return 2048.0 if synth.LINEARS_8B[layer][0] == "down" else 448.0


def dy_offset(step: int, view: int) -> int:
    """view 0: dY ROW, 1: dY COL H0, 2: dY COL H16."""
    return 8 * step + view


def f32hex(v) -> str:
    return "%08x" % int(np.asarray(v, dtype=np.float32).view(np.uint32))


def digest_row(x, amax, T, rounding="rne", offset=0):
    """Digests of the ROW view of x (payload, scales), its g and its health counts."""
    hq, hs = hashlib.sha256(), hashlib.sha256()
    g, sat, zero = None, 0, 0
    for r0 in range(0, x.shape[0], CHUNK):
        q = oracle.quantize_1d(x[r0:r0 + CHUNK], U, B, amax=amax, T=T, rounding=rounding, seed=SEED, offset=offset,
                               row0=r0)
        hq.update(np.ascontiguousarray(q.packed).tobytes())
        hs.update(np.ascontiguousarray(q.scales).tobytes())
        g, sat, zero = q.g, sat + q.n_sat, zero + q.n_zero
    return {"q": hq.hexdigest(), "s": hs.hexdigest(), "g": f32hex(g), "health": [sat, zero, 0]}


def digest_col(x, amax, T, hadamard_n, rounding="rne", offset=0):
    """Digests of the COL view (x^T, blocks along tokens, optional rotation) of x, its g and its
    health counts."""
    hq, hs = hashlib.sha256(), hashlib.sha256()
    g, sat, zero = None, 0, 0
    for f0 in range(0, x.shape[1], CHUNK):
        v = oracle.transposed_view(x[:, f0:f0 + CHUNK], hadamard_n)
        q = oracle.quantize_1d(v, U, B, amax=amax, T=T, rounding=rounding, seed=SEED, offset=offset, row0=f0)
        hq.update(np.ascontiguousarray(q.packed).tobytes())
        hs.update(np.ascontiguousarray(q.scales).tobytes())
        g, sat, zero = q.g, sat + q.n_sat, zero + q.n_zero
    return {"q": hq.hexdigest(), "s": hs.hexdigest(), "g": f32hex(g), "health": [sat, zero, 0]}


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _block(qa, qb, va="1d", vb="1d", hadamard_n=0):
    a, sa = oracle.operand_from_quant(qa, va)
    b, sb = oracle.operand_from_quant(qb, vb)
    return oracle.gemm_model(a, sa, b, sb, qa.block, alpha=oracle.output_scale(qa.g, qb.g, hadamard_n))


def sample_slices(n: int):
    return [(0, 8), (n - 8, n)]


def sample_cols(n: int):
    return [(0, 32), (n - 32, n)]


def gemm_samples(layer, step, X, dY, W, am):
    """Sampled blocks of fprop Y[tok, out], dgrad dX[tok, in] and wgrad dW[out, in] (H0 and H16),
    each from the oracle quantization of the slices it needs (the slices' own row offsets for
    the stochastic-rounding counters, 2D tiles aligned to 16, the whole tensors' cached amax)."""
    _, in_f, out_f = synth.LINEARS_8B[layer]
    tok, outs, ins = sample_slices(X.shape[0]), sample_cols(out_f), sample_cols(in_f)
    xr = [oracle.quantize_1d(X[a:b], U, B, amax=am["x"], T=T_X, row0=a) for a, b in tok]
    w_out = [oracle.quantize_2d(W[a:b], U, amax=am["w"], T=448.0) for a, b in outs]
    dyr = [oracle.quantize_1d(dY[a:b], U, B, amax=am["dy"], T=T_DY_ROW, rounding="sr", seed=SEED,
                              offset=dy_offset(step, 0), row0=a) for a, b in tok]
    w_in = [oracle.quantize_2d(W[:, a:b], U, amax=am["w"], T=448.0) for a, b in ins]
    out = {"fprop": np.block([[_block(xa, wb, vb="2d") for wb in w_out] for xa in xr]),
           "dgrad": np.block([[_block(da, wb, vb="2dT") for wb in w_in] for da in dyr])}
    for hn, key_x, key_dy, view in ((0, "x", "dy", 1), (16, "x16", "dy16", 2)):
        dyc = [oracle.quantize_1d(oracle.transposed_view(dY[:, a:b], hn), U, B, amax=am[key_dy], T=t_dy_col(layer),
                                  rounding="sr", seed=SEED, offset=dy_offset(step, view), row0=a) for a, b in outs]
        xc = [oracle.quantize_1d(oracle.transposed_view(X[:, a:b], hn), U, B, amax=am[key_x], T=T_X, row0=a)
              for a, b in ins]
        out[f"wgrad{hn}"] = np.block([[_block(da, xb, hadamard_n=hn) for xb in xc] for da in dyc])
    return {k: np.asarray(a, dtype=np.float32) for k, a in out.items()}


def main_task(args):
    """One (layer, checked step): inputs, amax samples, every view's digests, GEMM samples."""
    layer, step = args
    t0 = time.time()
    name, in_f, out_f = synth.LINEARS_8B[layer]
    tokens = synth.C5_TOKENS
    base = synth.layer_base(layer, tokens, in_f, out_f)
    amp = synth.step_amp(step)
    Xt = synth.drift_np(base["X"], synth.step_perm(layer, "X", step, tokens), amp)
    dYt = synth.drift_np(base["dY"], synth.step_perm(layer, "dY", step, tokens), amp)
    del base
    X, dY = Xt.values, dYt.values
    W = synth.layer_weight(layer, out_f, in_f).values
    res = {"layer": layer, "step": step, "X_in": sha(Xt.bits), "dY_in": sha(dYt.bits)}
    # amax observations (used only where a cache samples: steps 0 and 50)
    obs = {"x": oracle.tensor_amax(X), "x16": oracle.tensor_amax(X, 16), "dy": oracle.tensor_amax(dY),
           "dy16": oracle.tensor_amax(dY, 16), "w": oracle.tensor_amax(W)}
    res["obs"] = {k: f32hex(v) for k, v in obs.items()}
    # the caches hold the amax of the last sample step (0 or 50) of the same operand
    samp = 0 if step < D else D
    if samp == step:
        am = obs
    else:
        sb = synth.layer_base(layer, tokens, in_f, out_f)
        a_amp = synth.step_amp(samp)
        Xs = synth.drift_np(sb["X"], synth.step_perm(layer, "X", samp, tokens), a_amp).values
        dYs = synth.drift_np(sb["dY"], synth.step_perm(layer, "dY", samp, tokens), a_amp).values
        am = {"x": oracle.tensor_amax(Xs), "x16": oracle.tensor_amax(Xs, 16), "dy": oracle.tensor_amax(dYs),
              "dy16": oracle.tensor_amax(dYs, 16), "w": oracle.tensor_amax(W)}
        del sb, Xs, dYs
    v = {}
    v["x_row"] = digest_row(X, am["x"], T_X)
    v["x_col0"] = digest_col(X, am["x"], T_X, 0)
    v["x_col16"] = digest_col(X, am["x16"], T_X, 16)
    v["dy_row"] = digest_row(dY, am["dy"], T_DY_ROW, "sr", dy_offset(step, 0))
    v["dy_col0"] = digest_col(dY, am["dy"], t_dy_col(layer), 0, "sr", dy_offset(step, 1))
    v["dy_col16"] = digest_col(dY, am["dy16"], t_dy_col(layer), 16, "sr", dy_offset(step, 2))
    if step in (0, D):
        w2 = oracle.quantize_2d(W, U, amax=am["w"], T=448.0)
        v["w2d"] = {"q": sha(w2.packed), "qt": sha(oracle.pack_codes(np.ascontiguousarray(w2.codes.T))),
                    "s": sha(w2.scales), "g": f32hex(w2.g), "health": [w2.n_sat, w2.n_zero, 0]}
    res["views"] = v
    res["samples"] = gemm_samples(layer, step, X, dY, W, am)
    res["seconds"] = time.time() - t0
    return res


def stress_task(_):
    """The o projection with drift 1.12: caches, health counts of three views every step,
    digests at the steps around the headroom edges."""
    t0 = time.time()
    layer = STRESS_LAYER
    name, in_f, out_f = synth.LINEARS_8B[layer]
    tokens = synth.C5_TOKENS
    base = synth.layer_base(layer, tokens, in_f, out_f)
    cx, cdy = oracle.AmaxCache(D), oracle.AmaxCache(D)
    stats = {"x_row": [], "dy_row": [], "dy_col": []}
    caches = {"x": [], "dy": []}
    hashes = {}
    for step in range(synth.C5_STEPS):
        amp = synth.step_amp(step, STRESS_DRIFT)
        X = synth.drift_np(base["X"], synth.step_perm(layer, "X", step, tokens), amp).values
        dY = synth.drift_np(base["dY"], synth.step_perm(layer, "dY", step, tokens), amp).values
        Ax = cx.update(step, oracle.tensor_amax(X) if cx.needs_sample(step) else None)
        Ady = cdy.update(step, oracle.tensor_amax(dY) if cdy.needs_sample(step) else None)
        caches["x"].append(f32hex(Ax))
        caches["dy"].append(f32hex(Ady))
        stats["x_row"].append(list(oracle.block_health(X, U, B, amax=Ax, T=T_X)))
        stats["dy_row"].append(list(oracle.block_health(dY, U, B, amax=Ady, T=T_DY_ROW)))
        stats["dy_col"].append(list(oracle.block_health(dY, U, B, amax=Ady, T=2048.0, view="col")))
        if step in STRESS_HASH_STEPS["x_row"]:
            hashes[f"x_row@{step}"] = digest_row(X, Ax, T_X)
        if step in STRESS_HASH_STEPS["dy_col"]:
            hashes[f"dy_col@{step}"] = digest_col(dY, Ady, 2048.0, 0, "sr", dy_offset(step, 1))
    return {"stress": True, "stats": stats, "caches": caches, "hashes": hashes, "seconds": time.time() - t0}


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workers", type=int, default=6)
    args = ap.parse_args()
    import multiprocessing as mp
    tasks = [("stress", None)] + [("main", (l, s)) for l in range(len(synth.LINEARS_8B))
                                  for s in synth.C5_CHECK_STEPS]
    results = []
    t0 = time.time()
    with mp.get_context("fork").Pool(args.workers) as pool:
        jobs = [pool.apply_async(stress_task if kind == "stress" else main_task, (a,)) for kind, a in tasks]
        for j in jobs:
            r = j.get()
            results.append(r)
            what = "stress" if r.get("stress") else f"layer {r['layer']} step {r['step']}"
            print(f"{what}: {r['seconds']:.0f} s (elapsed {time.time() - t0:.0f} s)", flush=True)
    out = {"recipe": {"fmt": "ue5m3", "block": B, "D": D, "seed": SEED, "T_x": T_X, "T_dy_row": T_DY_ROW,
                      "T_dy_col": {n: t_dy_col(i) for i, (n, _, _) in enumerate(synth.LINEARS_8B)},
                      "tokens": synth.C5_TOKENS, "steps": synth.C5_STEPS, "check_steps": list(synth.C5_CHECK_STEPS),
                      "drift": 1.02, "dy_offsets": "8*step + view (0 ROW, 1 COL H0, 2 COL H16)",
                      "stress": {"layer": STRESS_LAYER, "drift": STRESS_DRIFT, "T_dy_col": 2048.0}},
           "layers": {}, "stress": None}
    arrays = {}
    obs_at = {}
    for r in results:
        if r.get("stress"):
            out["stress"] = {k: r[k] for k in ("stats", "caches", "hashes")}
            continue
        name = synth.LINEARS_8B[r["layer"]][0]
        lay = out["layers"].setdefault(name, {"steps": {}})
        lay["steps"][str(r["step"])] = {"X_in": r["X_in"], "dY_in": r["dY_in"], "views": r["views"]}
        obs_at[(name, r["step"])] = r["obs"]
        for k, a in r["samples"].items():
            arrays[f"{name}_s{r['step']}_{k}"] = a
    # cache sequences over all steps: samples at steps 0 and 50 (the only ones a D=50 cache takes)
    for name, lay in out["layers"].items():
        seqs = {}
        for key in ("x", "x16", "dy", "dy16", "w"):
            c = oracle.AmaxCache(D)
            seq = []
            for step in range(synth.C5_STEPS):
                if c.needs_sample(step):
                    c.update(step, np.uint32(int(obs_at[(name, step)][key], 16)).view(np.float32))
                seq.append(f32hex(c.amax))
            seqs[key] = seq
        lay["caches"] = seqs
    with open(JSON_OUT, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    np.savez_compressed(NPZ_OUT, **arrays)
    print(f"wrote {JSON_OUT} and {NPZ_OUT} in {time.time() - t0:.0f} s")


if __name__ == "__main__":
    main()
