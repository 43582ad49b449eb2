"""Throughput of the direct-ptychography hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-ssb-sweep]

Workload: the full-frame configuration (512 x 512 scan, 0.373 A step,
192 x 192 detector, 300 kV, 30 mrad soft aperture, 9298 bright-field pixels,
rotation 176.3 deg, 14 aberration terms, tilt (5.92, -0.07) mrad,
upsampling 3, G = (9298, 512, 257) complex64 = 9.8 GB, Poisson noise),
generated on the GPU with plain torch ops and resident in HBM before timing.

One step is one pass of the whole path over that G:
  phase prepare (pixel terms, transfer + Gram + right side, eigenbasis)
  + solve at one strength + scatter to the fine half plane,
  complex prepare (pixel terms, transfer + Gram + right side)
  + solve at one strength pair + scatter,
  SSB sum and agreement over the 0.2-0.9 1/A band for one optics set.

value = solved scan frequencies per step / seconds per step.  The line also
carries the phase prepare alone (the pages' headline stage), the G read
rate, the roofline of the dominant kernel (HIP events on the stream the
kernels run on), and the oracle's rate on a bounded sample of the same
workload on the host cores (cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "scan freqs/s for prepare (Gram+rhs+eigh) and G read GB/s, 512x512 scan"
UNIT = "scan freqs/s"

# MI355X published peaks
HBM_PEAK_GBPS = 8000.0
FP64_VECTOR_PEAK_TFLOPS = 78.6   # 256 CU x 4 SIMD x 16 lanes x 2 flop (FMA) x 2.4 GHz

# Algorithmic FP64 flops of the transfer + Gram kernel, per counted unit.
#   support test (pixel, alias, lobe): k -/+ Q (2), squared length (3)      = 5
#   non-zero lobe: theta = lambda k' + tau (2 FMA = 4), chi(theta) as a
#     degree-6 bivariate polynomial of 28 coefficients by Horner (27 FMA = 54),
#     phase difference (1), sine and cosine by the table method (reduction 1
#     FMA = 2, r^2 1, sine r - r^3/6 3, cosine to r^4 2 FMA = 4, angle
#     addition 2 MUL + 2 FMA = 6: 16), aperture product (1), amplitude times
#     cos and sin (2)                                                        = 78
#   non-zero column per pixel: weight times column (2), diagonal |t|^2 w
#     (2 FMA = 4), right side conj(t) w g (4 FMA = 8)                        = 14
#   non-zero column pair c < d per pixel: conj(t_c) w t_d (4 FMA)           = 8
#   (pixel, frequency) term: w g (2), power w |g|^2 (2 FMA = 4)              = 6
FLOP_TEST, FLOP_LOBE, FLOP_COL, FLOP_PAIR, FLOP_TERM = 5.0, 78.0, 14.0, 8.0, 6.0

KERNEL_SOURCES = ("stem_direct_ptychography_amd/csrc/dsp_kernels.hip",
                  "stem_direct_ptychography_amd/csrc/dsp_internal.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gram_full_frame.txt")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gram_flops(work: dict) -> float:
    return (FLOP_TEST * work["tests"] + FLOP_LOBE * work["lobes"] + FLOP_COL * work["cols"]
            + FLOP_PAIR * work["pairs"] + FLOP_TERM * work["terms"])


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed counter summary,
    or None when there is none or the kernel sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
    if kv.get("source_sha256_16") != kernel_source_hash() or kv.get("kernel") != kernel:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------
# workload
# ----------------------------------------------------------------------------


def build_inputs(dev):
    from synthetic import bf_pixels, data_stack_torch, workload

    w = workload("c4")
    pix, k = bf_pixels(w)
    log(f"generating G {(len(k), w.n_scan, w.n_half)} complex64 on {dev}")
    t = time.perf_counter()
    G = data_stack_torch(w, pix, dev)
    import torch

    torch.cuda.synchronize()
    log(f"G ready in {time.perf_counter() - t:.1f} s ({G.numel() * 8 / 1e9:.2f} GB)")
    return w, k, G


class Step:
    """One pass of the whole path; keeps the per-stage results of the last pass."""

    def __init__(self, dsp, w, k, G, band):
        self.dsp, self.w, self.k, self.G, self.band = dsp, w, k, G, band
        self.strength = 1e-2
        self.last = {}

    def __call__(self, timing: bool):
        dsp, w, k, G = self.dsp, self.w, self.k, self.G
        pp = dsp.prepare(G, k, w.optics, step=w.step, upsampling=w.upsampling, method="phase",
                         smoothness=w.smoothness, timing=timing)
        xp = pp.solve([self.strength])
        sp = pp.scatter(xp)
        pc = dsp.prepare(G, k, w.optics, step=w.step, upsampling=w.upsampling, method="complex",
                         smoothness=w.smoothness, timing=timing)
        xc = pc.solve([(self.strength, self.strength)])
        sc = pc.scatter(xc)
        S, Nn, E = dsp.ssb(G, k, [w.optics], step=w.step, band=self.band)
        self.last = {"phase": pp, "complex": pc, "outputs": (sp, sc, S, Nn), "E": E}
        return self.last


# ----------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on every host core
# ----------------------------------------------------------------------------
#
# A pool of spawned worker processes (the bench process holds a GPU context,
# so no fork), one BLAS thread each, runs the oracle's prepare + solve or SSB
# sum over chunks of frequencies whose G columns the parent has gathered.
# Wall clock of each pool run, data generation and gathering excluded.


def _oracle_prepare_chunk(args):
    """Worker: the oracle's prepare + solve of one chunk (compute seconds)."""
    from threadpoolctl import threadpool_limits

    from oracle import dsp_oracle as O
    from synthetic import workload

    name, method, q, cols, ka, wa, strengths = args
    w = workload(name)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        pr = O.prepare(q, [cols[:, i].astype(np.complex128) for i in range(cols.shape[1])], ka, wa, w.n_scan,
                       w.step, w.upsampling, w.optics, method, w.smoothness)
        for st in strengths:
            O.solve(pr, st)
        return time.perf_counter() - t0


def _oracle_ssb_chunk(args):
    """Worker: the oracle's SSB sums of one chunk of band entries."""
    from threadpoolctl import threadpool_limits

    from oracle import dsp_oracle as O
    from synthetic import ssb_sets, workload

    name, B, ent, cols, ka, wa = args
    w = workload(name)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.ssb(ent, [cols[:, i].astype(np.complex128) for i in range(cols.shape[1])], ka, wa, w.n_scan, w.step,
              ssb_sets(w, B))
        return time.perf_counter() - t0


def _gather(G, act_t, idx, dev):
    """complex64 (n_act, n) columns of G at stored indices idx (n, 2)."""
    import torch

    g = G[:, torch.as_tensor(idx[:, 0], device=dev), torch.as_tensor(idx[:, 1], device=dev)]
    return g[act_t].cpu().numpy()


def cpu_baseline(dsp, dev, w4, k4, G4, n_q: int, n_band: int, strength: float, workers: int):
    """The oracle on all host cores: C1 and C2 in full, seeded 2048-frequency
    samples of C3's sweep and of the full frame stratified by alias count
    (extrapolated per stratum), and the SSB sum on the band at 1 and 8 sets
    (sampled, extrapolated).  value = the full frame's step rate in scan frequencies/s
    (phase prepare + solve, complex prepare + solve, one-set SSB pass)."""
    import multiprocessing as mp

    import torch

    from oracle import dsp_oracle as O
    from synthetic import bf_pixels, data_stack_numpy, data_stack_torch, workload

    ctx = mp.get_context("spawn")
    out = {"kind": "oracle", "unit": UNIT, "cores": workers, "cpu_model": _cpu_model(),
           "affinity_cores": len(os.sched_getaffinity(0)), "configs": {}}
    pool = ctx.Pool(workers)
    try:
        pool.map(abs, range(4 * workers))   # the workers have started before any timing
        def run_prepare(name, G, k, method, strengths, q_idx, chunk):
            w = workload(name)
            act = O.active_pixels(k, w.optics)
            ka, wa = k[act], np.ones(len(act))
            act_t = torch.as_tensor(act, device=dev)
            Ga = None if isinstance(G, torch.Tensor) else G[act]
            jobs = []
            for c0 in range(0, len(q_idx), chunk):
                qc = q_idx[c0:c0 + chunk]
                cols = _gather(G, act_t, qc, dev) if Ga is None else Ga[:, qc[:, 0], qc[:, 1]]
                jobs.append((name, method, qc, cols, ka, wa, strengths))
            t0 = time.perf_counter()
            busy = pool.map(_oracle_prepare_chunk, jobs, chunksize=1)
            return time.perf_counter() - t0, busy, len(act)

        def stratified(w, n_take, seed):
            # a seeded sample of the unique frequencies, stratified by alias
            # count: {A: (frequencies with A aliases, sampled indices)}
            _, counts, _ = O.alias_table(w.n_scan, w.step, w.upsampling, w.optics)
            uq = O.unique_frequencies(w.n_scan)
            rng = np.random.default_rng(seed)
            strata = {}
            for A in np.unique(counts):
                idx = np.nonzero(counts == A)[0]
                take = max(16, int(round(n_take * len(idx) / len(uq))))
                strata[int(A)] = (len(idx), np.sort(rng.choice(idx, size=min(take, len(idx)), replace=False)))
            return uq, strata

        # C1 and C2 in full (their own methods and strength sweeps)
        for name in ("c1", "c2"):
            w = workload(name)
            pix, k = bf_pixels(w)
            G = data_stack_numpy(w, pix)
            q = O.unique_frequencies(w.n_scan)
            sts = list(w.strengths)
            wall, busy, n_act = run_prepare(name, G, k, w.method, sts, q, 64)
            out["configs"][name] = {"method": w.method, "n_q": len(q), "strengths": len(sts), "wall_s": wall,
                                    "q_per_s": len(q) / wall, "g_GBps": len(q) * n_act * 8 / wall / 1e9}
            log(f"cpu baseline {name}: {len(q)} frequencies ({w.method}, {len(sts)} strengths) in {wall:.1f} s")
            del G

        # C3: its 32-strength sweep on 2048 frequencies stratified by alias count
        w3 = workload("c3")
        pix3, k3 = bf_pixels(w3)
        G3 = data_stack_torch(w3, pix3, dev)
        torch.cuda.synchronize()
        uq3, strata3 = stratified(w3, 2048, 2048)
        cpu_full = wall_tot = 0.0
        for A, (n_all, idx) in strata3.items():
            wall, busy, n_act = run_prepare("c3", G3, k3, w3.method, list(w3.strengths), uq3[idx], 32)
            cpu_full += sum(busy) * n_all / len(idx)
            wall_tot += wall
        n3 = sum(len(v[1]) for v in strata3.values())
        out["configs"]["c3"] = {
            "method": w3.method, "n_q": len(uq3), "strengths": len(w3.strengths),
            "sample": f"{n3} of {len(uq3)} frequencies, stratified by alias count", "sample_wall_s": wall_tot,
            "extrapolated_s": cpu_full / workers, "q_per_s": len(uq3) / (cpu_full / workers)}
        log(f"cpu baseline c3: {n3} frequencies x {len(w3.strengths)} strengths in {wall_tot:.1f} s, "
            f"extrapolated {cpu_full / workers:.1f} s")
        del G3

        # full frame: 2048 frequencies stratified by alias count, per method
        uq, strata = stratified(w4, 2048, 4096)
        est = {}
        sample_n = sum(len(v[1]) for v in strata.values())
        for method in ("phase", "complex"):
            st = strength if method == "phase" else (strength, strength)
            cpu_full = 0.0
            wall_tot = 0.0
            for A, (n_all, idx) in strata.items():
                wall, busy, n_act = run_prepare("c4", G4, k4, method, [st], uq[idx], 32)
                cpu_full += sum(busy) * n_all / len(idx)
                wall_tot += wall
            est[method] = cpu_full / workers
            out["configs"]["c4_" + method] = {
                "sample": f"{sample_n} of {n_q} frequencies, stratified by alias count "
                          + ", ".join(f"{A}: {len(v[1])}" for A, v in strata.items()),
                "sample_wall_s": wall_tot, "extrapolated_s": est[method], "q_per_s": n_q / est[method],
                "g_GBps": n_q * n_act * 8 / est[method] / 1e9}
            log(f"cpu baseline c4 {method}: {sample_n} frequencies in {wall_tot:.1f} s, "
                f"full frame extrapolated {est[method]:.1f} s")

        # SSB on the band: 1 and 8 sets over a seeded sample of band entries
        w5 = workload("c5")
        pix5, k5 = bf_pixels(w5)
        G5 = data_stack_torch(w5, pix5, dev)
        torch.cuda.synchronize()
        act5 = O.active_pixels(k5, w5.optics)
        act5_t = torch.as_tensor(act5, device=dev)
        ent = np.argwhere(O.band_mask(w5.n_scan, w5.step, w5.band))
        for B, n_s in ((1, 1024), (8, 256)):
            sel = ent[np.sort(np.random.default_rng(B).choice(len(ent), size=n_s, replace=False))]
            jobs = [("c5", B, sel[c0:c0 + 32], _gather(G5, act5_t, sel[c0:c0 + 32], dev), k5[act5],
                     np.ones(len(act5))) for c0 in range(0, n_s, 32)]
            t0 = time.perf_counter()
            busy = pool.map(_oracle_ssb_chunk, jobs, chunksize=1)
            wall = time.perf_counter() - t0
            full = sum(busy) * len(ent) / n_s / workers
            est[f"ssb{B}"] = full
            out["configs"][f"c5_ssb_{B}"] = {
                "sample": f"{n_s} of {len(ent)} band entries (seeded uniform)", "sample_wall_s": wall,
                "extrapolated_s": full, "q_sets_per_s": len(ent) * B / full,
                "g_GBps": len(ent) * len(act5) * 8 / full / 1e9}
            log(f"cpu baseline ssb B={B}: {n_s} entries in {wall:.1f} s, band pass extrapolated {full:.2f} s")
        del G5
        torch.cuda.empty_cache()
    finally:
        pool.close()
        pool.join()
    step_s = est["phase"] + est["complex"] + est["ssb1"]
    out["value"] = n_q / step_s
    out["sample"] = (f"oracle on {workers} worker processes: c1 and c2 prepare + solve in full; c3's 32-strength "
                     f"sweep and the full frame's phase and complex prepare + solve on samples of 2048 frequencies "
                     f"stratified by alias count ({sample_n} of {n_q} for the full frame) and the SSB sum on 1024 "
                     f"(one set) and 256 (eight sets) of {n_band} band entries, each extrapolated to the whole "
                     f"workload; value = full-frame step rate (phase + complex + one-set SSB)")
    out["phase_prepare_q_per_s"] = n_q / est["phase"]
    return out


def cpu_full_frame(dev, workers: int):
    """The oracle's phase and complex prepare + solve over all 130,560
    frequencies of the full frame (not a sample), in batches of 8192 over the
    same worker pool; checks the stratified extrapolation that cpu_baseline
    reports.  One JSON line; minutes of host time, so not part of a default
    run."""
    import multiprocessing as mp

    import torch

    from oracle import dsp_oracle as O
    from synthetic import bf_pixels, data_stack_torch, workload

    w = workload("c4")
    pix, k = bf_pixels(w)
    log(f"generating G {(len(k), w.n_scan, w.n_half)} on {dev}")
    G = data_stack_torch(w, pix, dev)
    torch.cuda.synchronize()
    act = O.active_pixels(k, w.optics)
    ka, wa = k[act], np.ones(len(act))
    act_t = torch.as_tensor(act, device=dev)
    uq = O.unique_frequencies(w.n_scan)
    out = {"kind": "oracle", "workload": "c4 full frame, every frequency", "cores": workers,
           "cpu_model": _cpu_model(), "n_q": len(uq), "methods": {}}
    ctx = mp.get_context("spawn")
    pool = ctx.Pool(workers)
    try:
        pool.map(abs, range(4 * workers))
        for method, st in (("phase", 1e-2), ("complex", (1e-2, 1e-2))):
            busy_tot, t0 = 0.0, time.perf_counter()
            for b0 in range(0, len(uq), 8192):
                qb = uq[b0:b0 + 8192]
                jobs = [("c4", method, qb[c0:c0 + 32], _gather(G, act_t, qb[c0:c0 + 32], dev), ka, wa, [st])
                        for c0 in range(0, len(qb), 32)]
                busy_tot += sum(pool.map(_oracle_prepare_chunk, jobs, chunksize=1))
                log(f"oracle {method}: {b0 + len(qb)} of {len(uq)} frequencies")
            wall = time.perf_counter() - t0
            out["methods"][method] = {"wall_s": wall, "busy_per_worker_s": busy_tot / workers,
                                      "q_per_s": len(uq) / (busy_tot / workers)}
    finally:
        pool.close()
        pool.join()
    del G
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------------------
# SSB sweep over optics sets (the agreement workload: 8807 pixels, band pass)
# ----------------------------------------------------------------------------


def ssb_sweep(dsp, dev, reps: int = 5):
    import numpy as np
    import torch

    from synthetic import bf_pixels, data_stack_torch, ssb_sets, workload

    w = workload("c5")
    pix, k = bf_pixels(w)
    log(f"generating agreement-pass G {(len(k), w.n_scan, w.n_half)} on {dev}")
    G = data_stack_torch(w, pix, dev)
    n_band = dsp.band_count(w.n_scan, w.step, w.band)
    g_bytes = n_band * len(k) * 8.0
    out = {"workload": f"512x512 scan, {len(k)} BF px, band {w.band[0]}-{w.band[1]} 1/A ({n_band} stored q)",
           "g_bytes_per_pass": g_bytes, "passes": {}}
    stream = torch.cuda.current_stream()
    def timed(fn):
        fn()
        ms = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    # herm16 compact copies of the same stack (half the bytes per entry), one
    # scale per pixel or per stored row
    h16 = {"herm16": dsp.quantize_herm16(G), "herm16 rows": dsp.quantize_herm16(G, rows=True)}
    out["herm16_quantize_ms"] = timed(lambda: dsp.quantize_herm16(G))
    out["herm16_rows_quantize_ms"] = timed(lambda: dsp.quantize_herm16(G, rows=True))
    out["herm16_bytes"] = int(h16["herm16"][0].numel() * 2 + h16["herm16"][1].numel() * 4)
    out["herm16_rows_bytes"] = int(h16["herm16 rows"][0].numel() * 2 + h16["herm16 rows"][1].numel() * 4)
    out["complex64_bytes"] = int(G.numel() * 8)
    log(f"herm16 quantize: {out['herm16_quantize_ms']:.3f} ms, rows {out['herm16_rows_quantize_ms']:.3f} ms")
    # how far each compact copy moves the one-set SSB sums from complex64's
    S32, _, _ = dsp.ssb(G, k, ssb_sets(w, 1), step=w.step, band=w.band, agreement=False, want_N=False)
    for name, hq in h16.items():
        Sh, _, _ = dsp.ssb(None, k, ssb_sets(w, 1), step=w.step, band=w.band, agreement=False, want_N=False,
                           herm16=hq)
        out[name.replace(" ", "_") + "_rel_S_diff"] = float(torch.linalg.norm(Sh - S32) / torch.linalg.norm(S32))
        del Sh
    del S32
    # the pages' thick-sample fit batch: the same sets at depth 136 A
    runs = [(B, 0.0, None) for B in (1, 2, 4, 8)] + [(1, 136.0, None), (8, 136.0, None), (1, 0.0, "herm16"),
                                                      (8, 0.0, "herm16"), (1, 0.0, "herm16 rows"),
                                                      (8, 0.0, "herm16 rows")]
    for B, depth, packed in runs:
        sets = [o.replace(depth=depth) for o in ssb_sets(w, B)]
        if packed:
            m = timed(lambda: dsp.ssb(None, k, sets, step=w.step, band=w.band, agreement=False, herm16=h16[packed]))
        else:
            m = timed(lambda: dsp.ssb(G, k, sets, step=w.step, band=w.band, agreement=False))
        name = str(B) + ("" if depth == 0.0 else f" depth {depth:g} A") + (" " + packed if packed else "")
        gb = g_bytes / 2 if packed else g_bytes
        out["passes"][name] = {"ms": m, "q_sets_per_s": n_band * B / (m / 1e3), "g_GBps": gb / (m / 1e3) / 1e9}
        log(f"ssb B={name}: {m:.3f} ms")
    del G, h16
    torch.cuda.empty_cache()
    return out


def c3_sweep(dsp, dev, reps: int = 3):
    """The 256 x 256 strength sweep (phase method, upsampling 3): one prepare,
    then solve + scatter at each of its 32 strengths; stream time per stage,
    median over reps after one untimed call (layout built)."""
    import numpy as np
    import torch

    from synthetic import bf_pixels, data_stack_torch, workload

    w = workload("c3")
    pix, k = bf_pixels(w)
    log(f"generating sweep G {(len(k), w.n_scan, w.n_half)} on {dev}")
    G = data_stack_torch(w, pix, dev)
    sts = list(w.strengths)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    rows = []
    for r in range(reps + 1):
        ev[0].record(stream)
        p = dsp.prepare(G, k, w.optics, step=w.step, upsampling=w.upsampling, method="phase",
                        smoothness=w.smoothness)
        ev[1].record(stream)
        x = p.solve(sts)
        ev[2].record(stream)
        sc = p.scatter(x)
        ev[3].record(stream)
        torch.cuda.synchronize()
        if r:
            rows.append([ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]), ev[2].elapsed_time(ev[3])])
        n_q = p.info["n_q"]
        del p, x, sc
    med = np.median(np.asarray(rows), axis=0)
    total = float(med.sum())
    out = {"workload": f"256x256 scan, 0.373 A step, {len(k)} BF px, upsampling 3, phase method, "
                       f"{len(sts)} strengths (1e-3 .. 10)",
           "n_q": int(n_q), "strengths": len(sts), "prepare_ms": float(med[0]),
           "solve_all_strengths_ms": float(med[1]), "scatter_all_strengths_ms": float(med[2]),
           "total_ms": total, "q_per_s": n_q / (total / 1e3)}
    log(f"c3 sweep: {out}")
    del G
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------
# main
# ----------------------------------------------------------------------------


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (default: every core of this process's affinity set)")
    ap.add_argument("--no-ssb-sweep", action="store_true")
    ap.add_argument("--cpu-full-frame", action="store_true",
                    help="only time the oracle over every full-frame frequency (minutes of host time) and exit")
    ap.add_argument("--copy-probe", type=float, default=0.0,
                    help="only run a plain device copy of this many GiB (counter calibration) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the path shards by scan "
              f"frequency with no exchange; this build runs and reports a single GPU)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")

    if args.copy_probe > 0:
        n = int(args.copy_probe * (1 << 30)) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4}))
        return 0

    if args.cpu_full_frame:
        workers = args.cpu_workers or len(os.sched_getaffinity(0))
        print(json.dumps(cpu_full_frame(dev, workers)), flush=True)
        return 0

    import stem_direct_ptychography_amd as dsp

    log(f"library {dsp.LIB_PATH}")
    w, k, G = build_inputs(dev)
    band = (0.2, 0.9)
    step = Step(dsp, w, k, G, band)

    # work counts and flops per Gram launch (one instrumented prepare per method, untimed)
    flops = {}
    cold = {}
    for method in ("phase", "complex"):
        t0 = time.perf_counter()
        p = dsp.prepare(G, k, w.optics, step=w.step, upsampling=w.upsampling, method=method,
                        smoothness=w.smoothness, count_work=True)
        inf = p.timings()
        cold[method] = {"first_call_s": time.perf_counter() - t0, "layout_build_ms": inf["layout_ms"]}
        for g in inf["gram"]:
            flops[(method, g["nj"])] = (gram_flops(g["work"]), g["work"], g["tiles"])
        flops[(method, "lobes")] = inf["lobes"]
        del p
    torch.cuda.synchronize()

    for i in range(args.warmup):
        step(timing=True)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    stream = torch.cuda.current_stream()
    per = {"phase": [], "complex": []}
    gram_ms = {}
    fixup_ms = {}
    waves = {}
    host_ms = {"phase": [], "complex": []}
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        r = step(timing=True)
        for method in ("phase", "complex"):
            inf = r[method].timings()   # synchronizes the prepare's events (already passed)
            per[method].append(inf["stage_ms"])
            host_ms[method].append(inf["host_ms"])
            for g in inf["gram"]:
                gram_ms.setdefault((method, g["nj"]), []).append(g["ms"])
                fixup_ms.setdefault((method, g["nj"]), []).append(g["fixup_ms"])
                waves[(method, g["nj"])] = g["waves"]
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    log(f"{args.steps} steps: wall {wall:.3f} s, stream {gpu_ms:.1f} ms")
    ms_per_step = wall * 1e3 / args.steps

    inf_p = step.last["phase"].info
    n_q = inf_p["n_q"]
    g_bytes = inf_p["g_bytes"]
    n_band = dsp.band_count(w.n_scan, w.step, band)
    ssb_bytes = n_band * inf_p["n_active_bf"] * 8.0
    step_g_bytes = 2 * g_bytes + ssb_bytes

    def med(v):
        return float(np.median(v))

    stages = {}
    for method in ("phase", "complex"):
        s = np.array(per[method])
        stages[method] = {"pixel_terms_ms": med(s[:, 0]), "gram_ms": med(s[:, 1]), "eigenbasis_ms": med(s[:, 2]),
                          "prepare_kernels_ms": med(s[:, 3]), "host_geometry_ms": med(host_ms[method]),
                          "prepare_q_per_s": n_q / (med(s[:, 3]) / 1e3),
                          "prepare_g_GBps": g_bytes / (med(s[:, 3]) / 1e3) / 1e9}

    # dominant kernel: the Gram launch with the largest time per step
    launches = []
    for key, v in gram_ms.items():
        f, work, tiles = flops[key]
        m = float(np.mean(v))
        launches.append({"method": key[0], "slots": key[1], "tiles": tiles, "waves": waves[key], "avg_ms": m,
                         "fixup_ms": float(np.mean(fixup_ms[key])),
                         "flops": f, "tflops": f / (m / 1e3) / 1e12, "lobes": work["lobes"]})
    launches.sort(key=lambda d: -d["avg_ms"])
    dom = launches[0]
    kname = f"gram_kernel<{dom['slots']},{0 if dom['method'] == 'phase' else 1}>"
    tr = measured_traffic(kname)
    # algorithmic HBM bytes of the launch: one complex64 G value per (pixel, frequency) term
    alg_bytes = 8.0 * flops[(dom["method"], dom["slots"])][1]["terms"]
    roofline = {"bound": "alu", "achieved": dom["tflops"], "peak": FP64_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": dom["tflops"] / FP64_VECTOR_PEAK_TFLOPS, "traffic": tr,
                "alg_bytes": alg_bytes, "traffic_over_alg": (tr / alg_bytes) if tr else None,
                "kernel": f"{kname} ({dom['method']} Gram, tiles with {dom['slots']} alias slots, "
                          f"{dom['tiles']} tiles, {dom['lobes']:.3e} non-zero lobes per launch)",
                "avg_launch_ms": dom["avg_ms"], "flops_per_launch": dom["flops"]}
    gram_stage = {}
    for method in ("phase", "complex"):
        ls = [d for d in launches if d["method"] == method]
        tf = sum(d["flops"] for d in ls)
        tm = sum(d["avg_ms"] for d in ls)
        gram_stage[method] = {"ms": tm, "tflops": tf / (tm / 1e3) / 1e12,
                              "frac_fp64_peak": tf / (tm / 1e3) / 1e12 / FP64_VECTOR_PEAK_TFLOPS,
                              "g_GBps": g_bytes / (tm / 1e3) / 1e9,
                              "frac_hbm_peak": g_bytes / (tm / 1e3) / 1e9 / HBM_PEAK_GBPS,
                              "lobes": flops[(method, "lobes")]}

    result = {
        "metric": METRIC,
        "value": n_q / (ms_per_step / 1e3),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "full frame: 512x512 scan, 0.373 A step, 192x192 detector, 300 kV, 30 mrad soft, "
                               "9298 BF px, rot 176.3 deg, 14 aberrations, tilt (5.92,-0.07) mrad, upsampling 3, "
                               "G (9298,512,257) complex64; step = phase prepare+solve+scatter, complex "
                               "prepare+solve+scatter, SSB+agreement over the 0.2-0.9 1/A band",
                   "layout": "data-only layout (frequencies, aliases, tiles, priors, active pixels, stream-K "
                             "plans) built on the first prepare and reused by the timed steps; its build time "
                             "is reported in cold_first_prepare",
                   "n_q": n_q, "alias_hist": inf_p["alias_hist"][3:7], "n_active_bf": inf_p["n_active_bf"],
                   "strength": step.strength},
        "g_read_GBps": step_g_bytes / (ms_per_step / 1e3) / 1e9,
        "g_bytes_per_step": step_g_bytes,
        "phase_prepare_q_per_s": stages["phase"]["prepare_q_per_s"],
        "phase_prepare_g_GBps": stages["phase"]["prepare_g_GBps"],
        "stages": stages,
        "cold_first_prepare": cold,
        "gram_stage": gram_stage,
        "gram_launches": launches,
        "roofline": roofline,
        "stream_ms_per_step": gpu_ms / args.steps,
        "agreement": float(step.last["E"][0]),
    }
    # phase model derived from the last complex model (no pass over G), outside the step
    d_ms = []
    for _ in range(3):
        e0.record(stream)
        pd = step.last["complex"].derive_phase()
        e1.record(stream)
        torch.cuda.synchronize()
        d_ms.append(e0.elapsed_time(e1))
        del pd
    result["phase_derived_from_complex_ms"] = float(np.median(d_ms))
    # the same prepares with the depth of the pages' saved fit (12.4 nm), outside the step
    deep = w.optics.replace(depth=124.0)
    depth_ms = {}
    for method in ("phase", "complex"):
        ts = []
        for _ in range(3):
            p = dsp.prepare(G, k, deep, step=w.step, upsampling=w.upsampling, method=method,
                            smoothness=w.smoothness, timing=True)
            ts.append(p.timings()["stage_ms"][3])
            del p
        depth_ms[method + "_prepare_ms"] = float(np.median(ts))
    result["depth_124A"] = depth_ms
    log(f"depth 124 A prepares: {depth_ms}")
    # previews (spectrum + phase image) at 1x and 3x and the loss path, outside the step
    pv = {}
    for u in (1, 3):
        ts = []
        for _ in range(4):
            e0.record(stream)
            P, ph = dsp.preview(G, k, w.optics, step=w.step, upsampling=u)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
            del P, ph
        pv[f"preview_{u}x_ms"] = float(np.median(ts[1:]))
    ts = []
    for _ in range(3):
        e0.record(stream)
        mp, lv = dsp.loss(G, k, w.optics, step=w.step)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
        del mp
    pv["loss_path_ms"] = float(np.median(ts[1:]))
    pv["loss"] = lv
    result["preview"] = pv
    log(f"previews and loss path: {pv}")
    del step.last
    torch.cuda.synchronize()

    if not args.no_cpu_baseline:
        workers = args.cpu_workers or len(os.sched_getaffinity(0))
        log(f"timing the oracle on {workers} host cores")
        result["cpu_baseline"] = cpu_baseline(dsp, dev, w, k, G, n_q, n_band, step.strength, workers)
    else:
        result["cpu_baseline"] = None
    del G, step
    torch.cuda.empty_cache()
    if not args.no_ssb_sweep:
        result["ssb_sweep"] = ssb_sweep(dsp, dev)
        result["c3_sweep"] = c3_sweep(dsp, dev)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
