#!/usr/bin/env python3
"""Bench: PN decode-step GEMV weight-GB/s on one MI355X.

Workload (one step): one Qwen3.8-27B-shaped MLP at M = 1 token -- gate and up as pn3t 17408 x 5120,
down as pn4t 5120 x 17408. Gate and up read the same x, so they are stored stacked by rows as one
pn3t 34816 x 5120 matrix and run as one pn_gemv call (the usual fused gate/up projection); down is a
second call: two launches per step. Weights: seeded N(0, 0.02) fp32 quantized on the GPU by the
reference quantizer (pn_quantize_rows), checked against the CPU oracle's quantizer byte for byte on
every 97th row of each matrix before timing; one step's y is checked against the oracle on the same
rows after timing. x ~ N(0, 1) fp32. Five distinct device copies of the weight set (615.5 MB, above
the 256 MB Infinity Cache) are used round-robin, so every step reads its weights from HBM.
value = weight bytes per step / time per step.

Prints one JSON line (rank 0). See --help for the knobs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE, WRITE_SIZE), scaled by what
# the same counters read for a plain copy of known size; valid only for the kernel sources they
# were taken on (their hash is recorded with them).
COUNTERS_FILE = os.path.join(ROOT, "profiles", "pn_gemv_mlp_m1_hbm_counters.txt")
KERNEL_SOURCES = ["block_quantized_weight_pn3t_amd/csrc/pn_gemv_rows.hip",
                  "block_quantized_weight_pn3t_amd/csrc/pn_common.h"]
METRIC = "PN GEMV weight GB/s at M=1 (% of MI355X HBM peak), K=5120/17408"

# (name, type, [(rows, weight seed), ...] stacked by rows, K, x seed)
MLP = [("gate_up", 124, [(17408, 301), (17408, 302)], 5120, 304),
       ("down", 125, [(5120, 303)], 17408, 305)]


def host_threads() -> int:
    """Host threads for the oracle legs: the CPUs this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_weights(pn, torch, dev, copies):
    """Quantize each MLP matrix on the GPU and replicate it `copies` times in distinct buffers."""
    import numpy as np
    import synth
    mats = []
    for name, typ, parts, K, xseed in MLP:
        t0 = time.time()
        N = sum(n for n, _ in parts)
        rb = pn.row_bytes(typ, K)
        W0 = torch.empty((N, rb), dtype=torch.uint8, device=dev)
        st = torch.empty(N, dtype=torch.int32, device=dev)
        r0 = 0
        for n, wseed in parts:
            w = torch.from_numpy(synth.gaussian_weights(wseed, n, K, 0.02)).to(dev)
            pn.quantize_rows(typ, w, W0[r0:r0 + n], st[r0:r0 + n])
            del w
            r0 += n
        ver = torch.empty(N, dtype=torch.int32, device=dev)
        pn.validate_rows(typ, W0, N, K, ver)
        torch.cuda.synchronize()
        if int(st.abs().sum()) != 0 or int(ver.sum()) != N:
            raise RuntimeError(f"{name}: quantizer status / validation failed")
        oracle_check_bytes(name, typ, parts, K, W0)
        Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
        x = torch.from_numpy(np.ascontiguousarray(synth.activations(xseed, 1, K))).to(dev)
        y = torch.empty((1, N), dtype=torch.float32, device=dev)
        mats.append(dict(name=name, typ=typ, N=N, K=K, Ws=Ws, x=x, y=y, bytes=N * rb))
        log(f"[bench] {name}: {N}x{K} type {typ}, {N * rb / 1e6:.2f} MB x {copies} copies "
            f"({time.time() - t0:.1f} s)")
    return mats


SAMPLE_STRIDE = 97  # every 97th row of each matrix is checked against the oracle


def oracle_check_bytes(name, typ, parts, K, W0):
    """The GPU-quantized rows 0, 97, 194, ... of each stacked part must equal the CPU oracle's
    quantization of the same fp32 rows, byte for byte."""
    import numpy as np
    import oracle
    import synth
    r0 = 0
    for n, wseed in parts:
        rows = np.arange(0, n, SAMPLE_STRIDE)
        w = synth.gaussian_weights(wseed, n, K, 0.02)[rows]
        ref, st = oracle.quantize_rows(typ, np.ascontiguousarray(w), threads=host_threads())
        got = W0[r0 + rows].cpu().numpy()
        if st.any() or not np.array_equal(got, ref):
            raise RuntimeError(f"{name}: GPU quantizer differs from the oracle (seed {wseed})")
        r0 += n
    log(f"[bench] {name}: {sum(len(range(0, n, SAMPLE_STRIDE)) for n, _ in parts)} sampled rows "
        f"byte-identical to the oracle quantizer")


def oracle_check_step(mats):
    """One step's y on the sampled rows against the oracle: |y - y_ref| <= 1e-5 sum |w x|."""
    import numpy as np
    import oracle
    worst = 0.0
    for m in mats:
        rows = np.arange(0, m["N"], SAMPLE_STRIDE)
        W = m["Ws"][0][rows].cpu().numpy()
        x = m["x"].cpu().numpy()
        y = m["y"].cpu().numpy()[0, rows].astype(np.float64)
        y_ref, bound = oracle.gemv(m["typ"], np.ascontiguousarray(W), len(rows), m["K"], x,
                                   threads=host_threads())
        err = np.abs(y - y_ref[0])
        if not np.all(err <= 1e-5 * bound[0]):
            raise RuntimeError(f"{m['name']}: y outside the oracle bound")
        worst = max(worst, float(np.max(err / np.maximum(bound[0], 1e-300))))
    return worst


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kind: str):
    """HBM bytes per launch of `kind` from the counter summary, or None when there is none or it
    was taken on other kernel sources."""
    try:
        lines = open(COUNTERS_FILE).read().splitlines()
    except OSError:
        return None
    fields = {}
    for ln in lines:
        parts = ln.split()
        if len(parts) >= 2 and parts[0] in ("source_sha256", "traffic_bytes"):
            fields[(parts[0], parts[1] if parts[0] == "traffic_bytes" else "")] = parts[-1]
    if fields.get(("source_sha256", "")) != kernel_source_hash():
        return None
    v = fields.get(("traffic_bytes", kind))
    return int(v) if v is not None else None


def copy_calibration(torch, dev, mb: int, reps: int = 4):
    """Plain device copies of `mb` MiB (three rotated sources), for counter calibration: each copy
    reads and writes exactly mb MiB."""
    n = mb * (1 << 20) // 4
    srcs = [torch.full((n,), float(i + 1), dtype=torch.float32, device=dev) for i in range(3)]
    dst = torch.empty(n, dtype=torch.float32, device=dev)
    for i in range(reps):
        dst.copy_(srcs[i % 3])
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {mb} MiB")


# Untimed sustained work before each timed region: the GPU's clocks rise over the first
# milliseconds of back-to-back launches (the same launches run 20.5, 18.3 and 17.6 µs in three
# consecutive 6 ms windows after an idle host phase), and a decoder serving tokens runs in the
# settled state. Reported in the JSON line as settle_s.
SETTLE_S = 0.2


def settle(torch, launch, copies, seconds=SETTLE_S):
    """Run `launch(i)` back to back (rotating copies) for about `seconds` of wall time, untimed."""
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            launch(i % copies)
            i += 1
        torch.cuda.synchronize()


def time_launches(torch, stream, launch, copies, reps, warmup):
    """Average µs of `launch(i)` over `reps` back-to-back launches (rotating copies i % copies)
    between two events on the launch stream, after a settle phase and `warmup` launches."""
    settle(torch, launch, copies, SETTLE_S / 4)
    for i in range(warmup):
        launch(i % copies)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        launch(i % copies)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def check(st, what):
    if st != 0:
        raise RuntimeError(f"{what} failed: status {st}")


def quantize_pn(pn, torch, dev, typ, w_np):
    """Quantize fp32 rows on the GPU and validate them; returns the device bytes."""
    N, K = w_np.shape
    w = torch.from_numpy(w_np).to(dev)
    W = torch.empty((N, pn.row_bytes(typ, K)), dtype=torch.uint8, device=dev)
    st = torch.empty(N, dtype=torch.int32, device=dev)
    pn.quantize_rows(typ, w, W, st)
    ver = torch.empty(N, dtype=torch.int32, device=dev)
    pn.validate_rows(typ, W, N, K, ver)
    torch.cuda.synchronize()
    if int(st.abs().sum()) != 0 or int(ver.sum()) != N:
        raise RuntimeError("quantizer status / validation failed")
    return W


EXTRA_PARTS = ("pn4t6144", "layer", "nvfp4", "fp8row")


def extra_workloads(pn, torch, dev, reps, warmup, parts=EXTRA_PARTS):
    """The other measured configurations: per launch µs and weight-GB/s, weights rotated over
    enough copies to exceed the 256 MB Infinity Cache. parts selects which of them run."""
    import numpy as np
    import synth
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    out = {}

    def pn_entry(typ, N, K, Ws, M, x, y):
        us = time_launches(torch, stream, lambda c: check(pn.gemv_ptr(
            typ, Ws[c].data_ptr(), N, K, x.data_ptr(), M, y.data_ptr(), sh), "pn_gemv"),
            len(Ws), reps, warmup)
        return {"us": round(us, 3), "GBs": round(Ws[0].numel() / us / 1e3, 1)}

    if "pn4t6144" in parts:
        extra_pn4t6144(pn, torch, dev, reps, warmup, out, pn_entry)
    if "layer" in parts:
        extra_layer(pn, torch, dev, reps, warmup, out, pn_entry, stream, sh)
    if "nvfp4" in parts:
        extra_nvfp4(pn, torch, dev, reps, warmup, out, stream, sh)
    if "fp8row" in parts:
        extra_fp8row(pn, torch, dev, reps, warmup, out, stream, sh)
    return out


def extra_pn4t6144(pn, torch, dev, reps, warmup, out, pn_entry):
    import numpy as np
    import synth
    # pn4t 5120 x 6144, Laplace(0, 0.015) with 0.1% outliers x8, M = 1, 32 copies
    N, K = 5120, 6144
    W0 = quantize_pn(pn, torch, dev, 125, synth.laplace_outlier_weights(201, 202, N, K, 0.015, 0.001, 8.0))
    Ws = [W0] + [W0.clone() for _ in range(31)]
    x = torch.from_numpy(np.ascontiguousarray(synth.activations(203, 1, K))).to(dev)
    y = torch.empty((1, N), dtype=torch.float32, device=dev)
    out["pn4t_5120x6144_laplace_M1"] = pn_entry(125, N, K, Ws, 1, x, y)
    del Ws, W0
    log("[bench] extra: pn4t 5120x6144 done")


def extra_layer(pn, torch, dev, reps, warmup, out, pn_entry, stream, sh):
    import numpy as np
    import synth

    # decoder-layer set at M = 1..4, 4 copies (679.6 MB). Every layer figure is one layer's launches
    # issued back to back with copy c of every matrix at layer c, so consecutive layers rotate over
    # the whole 680 MB, past the 256 MB Infinity Cache. per_matrix_us times each matrix alone over
    # its own 4 copies, for reference: the small ones then fit the Infinity Cache.
    layer = [("gate", 124, 17408, 5120, 401), ("up", 124, 17408, 5120, 402), ("q", 124, 6144, 5120, 403),
             ("o", 124, 5120, 5120, 404), ("k", 125, 1024, 5120, 405), ("v", 125, 1024, 5120, 406),
             ("p6144", 125, 5120, 6144, 407), ("down", 125, 5120, 17408, 408)]
    C = 4
    mats = []
    for name, typ, N, K, seed in layer:
        W0 = quantize_pn(pn, torch, dev, typ, synth.gaussian_weights(seed, N, K, 0.02))
        mats.append((name, typ, N, K, [W0] + [W0.clone() for _ in range(C - 1)]))
    xs = {K: torch.from_numpy(np.ascontiguousarray(synth.activations(409, 4, K))).to(dev)
          for K in (5120, 6144, 17408)}
    xr = {K: torch.empty((4, K), dtype=torch.float32, device=dev) for K in xs}
    byname = {m[0]: m for m in mats}
    ys = {m[0]: torch.empty((4, m[2]), dtype=torch.float32, device=dev) for m in mats}
    set_bytes = sum(m[4][0].numel() for m in mats)
    order = ["q", "k", "v", "o", "gate", "up", "down", "p6144"]
    # the matrices that read one input (in the model: q, k, v; o; gate, up; down; the 6144-wide one)
    groups = [("q", "k", "v"), ("o",), ("gate", "up"), ("down",), ("p6144",)]
    garr = {g: [(pn.GemvPart * len(g))(*[pn.GemvPart(byname[n][1], byname[n][4][c].data_ptr(),
                                                      byname[n][2], ys[n].data_ptr()) for n in g])
                for c in range(C)] for g in groups if len(g) > 1}

    def plain(n, c, M, xsrc=None):
        _, typ, N, K, Ws = byname[n]
        check(pn.gemv_ptr(typ, Ws[c].data_ptr(), N, K, (xs[K] if xsrc is None else xsrc).data_ptr(),
                          M, ys[n].data_ptr(), sh), "pn_gemv")

    def layer_plain(c, M):
        for n in order:
            plain(n, c, M)

    def layer_grouped(c, M):
        for g in groups:
            if len(g) == 1:
                plain(g[0], c, M)
            else:
                K = byname[g[0]][3]
                check(pn.gemv_group_ptr(garr[g][c], K, xs[K].data_ptr(), M, sh), "pn_gemv_group")

    def layer_fused(c, M):
        for n in order:
            _, typ, N, K, Ws = byname[n]
            check(pn.gemv_hadamard_ptr(typ, Ws[c].data_ptr(), N, K, xs[K].data_ptr(), M, 1024,
                                       ys[n].data_ptr(), sh), "pn_gemv_hadamard")

    def layer_fused_grouped(c, M):
        for g in groups:
            K = byname[g[0]][3]
            if len(g) == 1:
                n = g[0]
                check(pn.gemv_hadamard_ptr(byname[n][1], byname[n][4][c].data_ptr(), byname[n][2],
                                           K, xs[K].data_ptr(), M, 1024, ys[n].data_ptr(), sh),
                      "pn_gemv_hadamard")
            else:
                check(pn.gemv_group_hadamard_ptr(garr[g][c], K, xs[K].data_ptr(), M, 1024, sh),
                      "pn_gemv_group_hadamard")

    def layer_rotate_once(c, M):
        for g in groups:
            K = byname[g[0]][3]
            check(pn.lib().pn_hadamard_rows(xs[K].data_ptr(), M, K, 1024, xr[K].data_ptr(), sh),
                  "pn_hadamard_rows")
            if len(g) == 1:
                plain(g[0], c, M, xr[K])
            else:
                check(pn.gemv_group_ptr(garr[g][c], K, xr[K].data_ptr(), M, sh), "pn_gemv_group")

    def layer_entry(fn, M, **kw):
        us = time_launches(torch, stream, lambda c: fn(c, M), C, reps, warmup)
        return {"GBs": round(set_bytes / us / 1e3, 1), "us": round(us, 2), **kw}

    for M in (1, 2, 3, 4):
        per = {n: pn_entry(byname[n][1], byname[n][2], byname[n][3], byname[n][4], M,
                           xs[byname[n][3]], ys[n])["us"] for n in order}
        out[f"layer_set_M{M}"] = layer_entry(layer_plain, M, per_matrix_us=per)
        out[f"layer_set_grouped_M{M}"] = layer_entry(layer_grouped, M)
    log("[bench] extra: layer set done")

    # Hadamard-rotated activations (slices of 1024): every matrix through pn_gemv_hadamard (the
    # rotation fused into each launch); the matrices that share an input through
    # pn_gemv_group_hadamard (one launch, the rotation fused); each distinct input rotated once
    # with pn_hadamard_rows and shared by the grouped launches; and the rotation on its own
    for M in (1, 2, 3, 4):
        out[f"hadamard1024_layer_set_M{M}"] = layer_entry(layer_fused, M)
        out[f"hadamard1024_layer_set_fused_grouped_M{M}"] = layer_entry(layer_fused_grouped, M)
        out[f"hadamard1024_layer_set_rotate_once_M{M}"] = layer_entry(layer_rotate_once, M)
    rot = {}
    for M in (1, 2, 3, 4):
        for K in (5120, 6144, 17408):
            rot[M, K] = time_launches(torch, stream, lambda c: check(pn.lib().pn_hadamard_rows(
                xs[K].data_ptr(), M, K, 1024, xr[K].data_ptr(), sh), "pn_hadamard_rows"), 1, reps,
                warmup)
    out["hadamard_rows_1024_us"] = {f"M{M}_K{K}": round(v, 3) for (M, K), v in rot.items()}
    del mats, garr, ys
    log("[bench] extra: Hadamard done")


def extra_nvfp4(pn, torch, dev, reps, warmup, out, stream, sh):
    import numpy as np
    import synth

    # NVFP4 17408 x 5120, clip-search quantized by the oracle (host threads), x bf16, M = 1..4,
    # 11 copies
    import oracle
    N, K = 17408, 5120
    w_np = synth.gaussian_weights(501, N, K, 0.02)
    gv = oracle.nvfp4_global_scale(w_np)
    c_np, s_np = oracle.nvfp4_quantize_rows(w_np, gv, threads=host_threads())
    del w_np
    codes = torch.from_numpy(c_np).to(dev)
    scales = torch.from_numpy(s_np).to(dev)
    C = [(codes, scales)] + [(codes.clone(), scales.clone()) for _ in range(10)]
    xb = torch.from_numpy(np.ascontiguousarray(synth.activations_bf16(502, 4, K)).view(np.int16)).to(dev)
    nbytes = codes.numel() + scales.numel() + 4
    yn = torch.empty((4, N), dtype=torch.float32, device=dev)  # y of up to 4 tokens
    for M in (1, 2, 3, 4):
        us = time_launches(torch, stream, lambda c: check(pn.gemv_nvfp4_ptr(
            C[c][0].data_ptr(), C[c][1].data_ptr(), gv, N, K, xb.data_ptr(), M, yn.data_ptr(), sh),
            "pn_gemv_nvfp4"), len(C), reps, warmup)
        out[f"nvfp4_17408x5120_M{M}"] = {"us": round(us, 3), "GBs": round(nbytes / us / 1e3, 1)}
    log("[bench] extra: nvfp4 done")
    del C, codes, scales


def extra_fp8row(pn, torch, dev, reps, warmup, out, stream, sh):
    import numpy as np
    import synth

    # row-scaled E4M3 head, 248,320 x 5,120 (1.27 GB of codes per copy): seeded valid E4M3FN words
    # and positive bf16 multipliers, 2 copies, M = 1..4
    N, K = 248320, 5120
    hc = torch.empty((N, K), dtype=torch.uint8, device=dev)
    hs = torch.empty(N, dtype=torch.int16, device=dev)
    for r0 in range(0, N, 16384):
        n = min(16384, N - r0)
        c_np, s_np = synth.e4m3_row_words(601 + r0, n, K)
        hc[r0:r0 + n] = torch.from_numpy(c_np).to(dev)
        hs[r0:r0 + n] = torch.from_numpy(s_np.view(np.int16)).to(dev)
    torch.cuda.synchronize()
    H = [(hc, hs), (hc.clone(), hs.clone())]
    xh = torch.from_numpy(np.ascontiguousarray(synth.activations(602, 4, K))).to(dev)
    yh = torch.empty((4, N), dtype=torch.float32, device=dev)
    hbytes = N * K + 2 * N
    for M in (1, 2, 3, 4):
        us = time_launches(torch, stream, lambda c: check(pn.gemv_fp8row_ptr(
            H[c][0].data_ptr(), H[c][1].data_ptr(), N, K, xh.data_ptr(), M, yh.data_ptr(), sh),
            "pn_gemv_fp8row"), len(H), max(10, reps // 10), max(2, warmup // 5))
        out[f"fp8row_head_248320x5120_M{M}"] = {"us": round(us, 2), "GBs": round(hbytes / us / 1e3, 1)}
    log("[bench] extra: fp8row head done")


def shard_shapes(pn, torch, dev, mats, reps, warmup):
    """One GPU's share of the MLP step at M = 1 when G = 2, 4, 8 GPUs share it: gate+up split by
    rows (G slices of N/G rows of the stacked 34816x5120 pn3t; no reduction), down split along K
    at block boundaries (5120 x 17408/G pn4t, a partial y per GPU for one all-reduce). Every
    slice of every rotated copy is its own buffer (> 256 MB in rotation). Launch-to-launch µs of
    the two launches and of each alone; the collective and the x broadcast are not part of it."""
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    gu, dn = mats
    out = {}
    for G in (2, 4, 8):
        n_gu = gu["N"] // G
        nb_dn = dn["K"] // 64 // G
        k_dn = nb_dn * 64
        gu_sh = [W[g * n_gu:(g + 1) * n_gu] for W in gu["Ws"] for g in range(G)]
        dn_sh = [W.view(dn["N"], -1, 34)[:, g * nb_dn:(g + 1) * nb_dn].contiguous()
                 for W in dn["Ws"] for g in range(G)]
        x_dn = dn["x"][:, :k_dn].contiguous()
        b_gu, b_dn = gu_sh[0].numel(), dn_sh[0].numel()

        def l_gu(c):
            check(pn.gemv_ptr(124, gu_sh[c].data_ptr(), n_gu, gu["K"], gu["x"].data_ptr(), 1,
                              gu["y"].data_ptr(), sh), "pn_gemv")

        def l_dn(c):
            check(pn.gemv_ptr(125, dn_sh[c].data_ptr(), dn["N"], k_dn, x_dn.data_ptr(), 1,
                              dn["y"].data_ptr(), sh), "pn_gemv")

        def step(c):
            l_gu(c)
            l_dn(c)
        n = len(gu_sh)
        us = time_launches(torch, stream, step, n, reps, warmup)
        us_gu = time_launches(torch, stream, l_gu, n, reps, warmup)
        us_dn = time_launches(torch, stream, l_dn, n, reps, warmup)
        out[f"G{G}"] = {"gate_up": f"{n_gu}x{gu['K']} pn3t", "down": f"{dn['N']}x{k_dn} pn4t",
                        "step_us": round(us, 3), "GBs": round((b_gu + b_dn) / us / 1e3, 1),
                        "gate_up_us": round(us_gu, 3), "gate_up_GBs": round(b_gu / us_gu / 1e3, 1),
                        "down_us": round(us_dn, 3), "down_GBs": round(b_dn / us_dn / 1e3, 1)}
        del gu_sh, dn_sh
    log("[bench] extra: shard shapes done")
    return out


def cpu_baseline(seconds: float):
    """The CPU oracle's GEMV timed on the host cores: a bounded sample (1/16 of the rows of each MLP
    matrix, quantized by the oracle), repeated to ~`seconds` of work."""
    import numpy as np
    import oracle
    import synth
    threads = max(1, min(16, os.cpu_count() or 1))
    samples = []
    for name, typ, parts, K, xseed in MLP:
        for N, wseed in parts:
            n = N // 16
            w = synth.gaussian_weights(wseed, N, K, 0.02)[:n]
            W, _ = oracle.quantize_rows(typ, w, threads=threads)
            samples.append((typ, n, K, W, synth.activations(xseed, 1, K), W.nbytes))
    def rate(nthreads, budget):
        total_bytes, reps, t0 = 0, 0, time.perf_counter()
        while True:
            for typ, n, K, W, x, nbytes in samples:
                oracle.gemv(typ, W, n, K, x, threads=nthreads)
                total_bytes += nbytes
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 1000:
                return total_bytes / el / 1e9, reps, el

    value, reps, el = rate(threads, seconds)
    one, reps1, el1 = rate(1, max(1.0, seconds / 6))  # the same sample on one thread
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(value, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..N/16 of each of gate, up, down (M=1), {reps} passes, {el:.1f} s, "
                      f"fp64 accumulation, {threads} host threads",
            "value_one_thread": round(one, 4),
            "sample_one_thread": f"the same sample, {reps1} passes, {el1:.1f} s, 1 host thread",
            "host": f"{cpu}; {os.cpu_count()} logical CPUs"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=5, help="rotated weight copies (>= 3 to exceed MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU-baseline budget (0 = skip)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other measured configurations (pn4t 5120x6144, layer set at "
                         "M=1..4, the layer set with Hadamard-rotated x at M=1..4, NVFP4 at M=1..4, "
                         "row-scaled E4M3 head at M=1..4)")
    ap.add_argument("--extra", default=",".join(EXTRA_PARTS),
                    help="which other configurations run (comma list of " + ", ".join(EXTRA_PARTS) +
                         "; the one-GPU shares of the MLP run with any of them)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="also run plain copies of this many MiB (counter calibration under rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this bench measures one GPU only: run with --gpus 1 "
                          "(the GEMV shards by rows, with no new kernels; several GPUs are not measured)"}))
        sys.exit(2)

    import torch
    import block_quantized_weight_pn3t_amd as pn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mats = build_weights(pn, torch, dev, args.copies)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    step_bytes = sum(m["bytes"] for m in mats)

    def one_step(s, evs=None):
        c = s % args.copies
        for j, m in enumerate(mats):
            if evs is not None:
                evs[j][0].record(stream)
            st = pn.gemv_ptr(m["typ"], m["Ws"][c].data_ptr(), m["N"], m["K"], m["x"].data_ptr(),
                             1, m["y"].data_ptr(), sh)
            if evs is not None:
                evs[j][1].record(stream)
            if st != 0:
                raise RuntimeError(f"pn_gemv failed: {pn.status_string(st)}")

    settle(torch, one_step, args.copies)
    for s in range(args.warmup):
        one_step(s)
    torch.cuda.synchronize()

    # timed region: K steps back to back on one stream, events only at the two ends
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        one_step(s)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    one_step(0)  # copy 0, outside the timed region
    torch.cuda.synchronize()
    check_worst = oracle_check_step(mats)
    log(f"[bench] one step's y on the sampled rows within the oracle bound (worst err/bound "
        f"{check_worst:.2e})")

    # per-kernel durations, live, on the launch stream: each kernel launched K times back to back
    # over the rotated copies between two events (avg = elapsed / K, launch gaps included), and
    # again with an event pair around every launch (marker overhead included).
    kern = {}
    for j, m in enumerate(mats):
        def launch(s, m=m):
            st = pn.gemv_ptr(m["typ"], m["Ws"][s % args.copies].data_ptr(), m["N"], m["K"],
                             m["x"].data_ptr(), 1, m["y"].data_ptr(), sh)
            if st != 0:
                raise RuntimeError(f"pn_gemv failed: {pn.status_string(st)}")
        settle(torch, launch, args.copies)
        for s in range(args.warmup):
            launch(s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.steps):
            launch(s)
        e1.record(stream)
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(args.steps)]
        for s in range(args.steps):
            pairs[s][0].record(stream)
            launch(s)
            pairs[s][1].record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        us_pair = sum(a.elapsed_time(b) for a, b in pairs) * 1e3 / args.steps
        kern[m["name"]] = dict(avg_us=round(us, 3), weight_GBs=round(m["bytes"] / us / 1e3, 1),
                               avg_us_event_pair=round(us_pair, 3), bytes=m["bytes"])
    # dominant kernel: the largest share of the step's kernel time, per kernel kind
    kinds = {"pn3t_34816x5120": ["gate_up"], "pn4t_5120x17408": ["down"]}
    tot = {k: sum(kern[n]["avg_us"] for n in v) for k, v in kinds.items()}
    dom = max(tot, key=tot.get)
    dnames = kinds[dom]
    d_bytes = kern[dnames[0]]["bytes"]
    d_us = sum(kern[n]["avg_us"] for n in dnames) / len(dnames)
    achieved = d_bytes / d_us / 1e3
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Qwen3.8-27B-shaped MLP at M=1: gate and up pn3t 17408x5120 each, "
                               "stacked as one 34816x5120 launch, down pn4t 5120x17408 "
                               "(2 pn_gemv launches per step)",
                   "weight_bytes_per_step": step_bytes, "rotated_copies": args.copies,
                   "working_set_MB": round(step_bytes * args.copies / 1e6, 1),
                   "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "kernel": f"pn_gemv {dom} (M=1)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dom),
                     "avg_launch_us": round(d_us, 3), "algorithmic_bytes_per_launch": d_bytes},
        "kernels": kern,
    }
    if not args.no_extra:
        parts = tuple(p for p in args.extra.split(",") if p)
        bad = [p for p in parts if p not in EXTRA_PARTS]
        if bad:
            raise SystemExit(f"unknown --extra part(s): {bad}")
        result["extra"] = extra_workloads(pn, torch, dev, args.steps, args.warmup, parts)
        result["extra"]["mlp_shard_M1"] = shard_shapes(pn, torch, dev, mats, args.steps,
                                                       args.warmup)
    if args.copy_mb > 0:
        copy_calibration(torch, dev, args.copy_mb)
    if args.cpu_seconds > 0:
        log("[bench] timing the CPU oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
