"""Seeded synthetic inputs for the direct-ptychography hot path.

This module is the only code shared by the CPU oracle (``oracle/``) and the
HIP library's callers (tests, ``bench.py``).  It holds no arithmetic of the
method itself: no aperture, no aberration phase, no transfer, no alias rule.
It only draws numbers:

* the workload descriptions (scan size, step, detector sampling, optics
  parameters, upsampling, method, strengths) of the five synthetic
  configurations;
* detector pixel coordinates of the bright-field candidates (a disk of
  pixels, or the n nearest pixels, rotated into the scan frame);
* seeded aberration coefficient draws and per-set perturbations;
* a seeded object contrast map on the scan grid;
* the measured-data stack G(q, k): the half-plane scan-space FFT of a stack of
  non-negative per-pixel intensity images, optionally Poisson sampled.

The intensity images are *not* produced by a physical forward model: each
bright-field pixel sees a brightness times (1 + 2 x a shifted copy of the
object contrast map).  That gives G the dynamic range of a measurement
(a dominant DC term, structured low-frequency content, a noise floor) and
the Hermitian symmetry of a real intensity stack, which is all the hot path
depends on: its cost depends on geometry only, and its results are linear in
G.  The physical weak-object forward models live in the oracle and are used by
the oracle's own pins.

Pages followed for the workloads: "Where the 9 s of regularized preparation
goes" (Setup: 512 x 512 scan, 0.373 A step, 192 x 192 detector, 300 kV,
30 mrad, rotation 176.3 deg, 14 aberration terms, tilt (5.92, -0.07) mrad,
upsampling 3, 9298 bright-field pixels) and "Tilt-corrected SSB on CUDA"
(Setup: 8,807 bright-field pixels, fit band 0.2 to 0.9 1/A).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# physical constants used to state the workloads
# ----------------------------------------------------------------------------


def electron_wavelength_A(kv: float) -> float:
    """Relativistic electron wavelength (A) at accelerating voltage ``kv``.

    lambda = h / sqrt(2 m0 e V (1 + e V / (2 m0 c^2))), CODATA constants.
    300 kV gives 0.0196875 A (the workloads quote 0.01969 A).
    """
    h = 6.62607015e-34
    m0 = 9.1093837015e-31
    e = 1.602176634e-19
    c = 299792458.0
    v = kv * 1e3
    p = math.sqrt(2.0 * m0 * e * v * (1.0 + e * v / (2.0 * m0 * c * c)))
    return h / p * 1e10


# The fourteen Krivanek (n, m) pairs of radial orders 1..5 with n+1-m even.
KRIVANEK_PAIRS: Tuple[Tuple[int, int], ...] = (
    (1, 0), (1, 2), (2, 1), (2, 3), (3, 0), (3, 2), (3, 4),
    (4, 1), (4, 3), (4, 5), (5, 0), (5, 2), (5, 4), (5, 6),
)


@dataclasses.dataclass
class Optics:
    """Probe optics.  Angles in rad, lengths in A, frequencies in 1/A.

    ``aberrations`` holds (n, m, C_nm [A], phi_nm [rad]) in Krivanek polar
    notation; ``tilt`` is (tau_y, tau_x) in rad; ``det_step`` is the detector
    pixel pitch in the scan frame (1/A).
    """

    wavelength: float
    semiangle: float
    det_step: float
    soft: bool = True
    tilt: Tuple[float, float] = (0.0, 0.0)
    aberrations: List[Tuple[int, int, float, float]] = dataclasses.field(default_factory=list)
    depth: float = 0.0

    def replace(self, **kw) -> "Optics":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass
class Workload:
    name: str
    n_scan: int
    step: float
    n_det: int
    optics: Optics
    upsampling: int
    bf_radius_px: Optional[float] = None   # candidates with |p - c| <= radius
    bf_nearest: Optional[int] = None       # or the n nearest pixels, order (r^2, iy, ix)
    rotation_deg: float = 0.0
    method: str = "phase"
    strengths: Sequence = ()
    dose: Optional[float] = None           # e/A^2; None: noise-free
    lattice_sites: int = 0                 # object: sites per axis (0: filtered white noise)
    smoothness: float = 0.0                # prior frequency s_p (1/A); <= 0: no prior
    band: Optional[Tuple[float, float]] = None
    n_sets: int = 1
    seed: int = 0

    @property
    def n_half(self) -> int:
        return self.n_scan // 2 + 1


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

LAMBDA_300KV = electron_wavelength_A(300.0)
ALPHA_30MRAD = 0.030


def _order_scaled_aberrations(rng: np.random.Generator, lam: float, alpha: float) -> List[Tuple[int, int, float, float]]:
    """14 Krivanek terms whose edge phase decays with radial order.

    For order n the phase the term reaches at the aperture edge is
    rho_n * U(0.5, 1) rad, rho = (10, 3, 1, 0.3, 0.1) for n = 1..5, which
    fixes |C_nm| = phase * (n + 1) * lambda / (2 pi alpha^(n+1)).  m = 0
    terms get a random sign, m > 0 terms a random angle in [0, 2 pi / m).
    """
    rho = {1: 10.0, 2: 3.0, 3: 1.0, 4: 0.3, 5: 0.1}
    out = []
    for n, m in KRIVANEK_PAIRS:
        phase = rho[n] * rng.uniform(0.5, 1.0)
        c = phase * (n + 1) * lam / (2.0 * math.pi * alpha ** (n + 1))
        if m == 0:
            c *= rng.choice([-1.0, 1.0])
            phi = 0.0
        else:
            phi = rng.uniform(0.0, 2.0 * math.pi / m)
        out.append((n, m, float(c), float(phi)))
    return out


def workload(name: str) -> Workload:
    """The five synthetic workloads (c1..c5) and small test variants."""
    lam, alpha = LAMBDA_300KV, ALPHA_30MRAD
    kc = alpha / lam
    name = name.lower()
    if name == "c1":
        # 32x32 scan, 0.5 A, 24x24 detector, hard 30 mrad aperture of radius
        # 6.04 px (113 pixels), defocus only, upsampling 1, noise-free.
        opt = Optics(lam, alpha, kc / 6.04, soft=False, aberrations=[(1, 0, -100.0, 0.0)])
        return Workload("c1", 32, 0.5, 24, opt, 1, bf_radius_px=6.04, method="phase",
                        strengths=(1e-3,), dose=None, lattice_sites=0, smoothness=kc, seed=1001)
    if name == "c2":
        rng = np.random.default_rng(np.random.SeedSequence(1002).spawn(3)[1])
        c10 = rng.uniform(-200.0, 200.0)
        c12 = rng.uniform(0.0, 50.0)
        phi12 = rng.uniform(0.0, math.pi)
        opt = Optics(lam, alpha, kc / 17.4, soft=True,
                     aberrations=[(1, 0, float(c10), 0.0), (1, 2, float(c12), float(phi12)), (3, 0, 1.0e4, 0.0)])
        return Workload("c2", 128, 0.4, 64, opt, 2, bf_radius_px=17.9, method="complex",
                        strengths=tuple((float(v), float(v)) for v in np.logspace(-3, 0, 8)),
                        dose=1e4, lattice_sites=16, smoothness=kc, seed=1002)
    if name in ("c3", "c4", "c5"):
        rng = np.random.default_rng(np.random.SeedSequence(1003).spawn(3)[1])
        aber = _order_scaled_aberrations(rng, lam, alpha)
        tilt = (5.92e-3, -0.07e-3)
        if name == "c3":
            opt = Optics(lam, alpha, kc / 35.6, soft=True, tilt=tilt, aberrations=aber)
            return Workload("c3", 256, 0.373, 128, opt, 3, bf_radius_px=36.1, method="phase",
                            strengths=tuple(float(v) for v in np.logspace(-3, 1, 32)),
                            dose=None, lattice_sites=30, smoothness=kc, seed=1003)
        opt = Optics(lam, alpha, 0.02819, soft=True, tilt=tilt, aberrations=aber)
        if name == "c4":
            return Workload("c4", 512, 0.373, 192, opt, 3, bf_nearest=9298, rotation_deg=176.3,
                            method="phase", strengths=(1e-2,), dose=1e5, lattice_sites=60,
                            smoothness=kc, seed=1004)
        return Workload("c5", 512, 0.373, 192, opt, 1, bf_nearest=8807, rotation_deg=176.3,
                        method="ssb", dose=1e5, lattice_sites=60, band=(0.2, 0.9), n_sets=8,
                        seed=1005)
    raise ValueError(f"unknown workload {name!r}")


def ssb_sets(w: Workload, n_sets: int) -> List[Optics]:
    """Optics sets for one agreement pass: set 0 is the workload's optics,
    sets 1.. perturb defocus (+-20 A), astigmatism (|C12| x (1 +- 0.1),
    angle +- 0.1 rad), spherical aberration (C30 x (1 +- 0.05)) and tilt
    (+-0.5 mrad per axis).  Sets are nested: the first n of 8 are the same
    for any n."""
    rng = np.random.default_rng(np.random.SeedSequence(w.seed).spawn(3)[1])
    out = [w.optics]
    for _ in range(1, 8):
        d10 = rng.uniform(-20.0, 20.0)
        f12 = 1.0 + rng.uniform(-0.1, 0.1)
        d12 = rng.uniform(-0.1, 0.1)
        f30 = 1.0 + rng.uniform(-0.05, 0.05)
        dty, dtx = rng.uniform(-0.5e-3, 0.5e-3, size=2)
        ab = []
        for (n, m, c, phi) in w.optics.aberrations:
            if (n, m) == (1, 0):
                c = c + d10
            elif (n, m) == (1, 2):
                c, phi = c * f12, phi + d12
            elif (n, m) == (3, 0):
                c = c * f30
            ab.append((n, m, float(c), float(phi)))
        t = (w.optics.tilt[0] + float(dty), w.optics.tilt[1] + float(dtx))
        out.append(w.optics.replace(aberrations=ab, tilt=t))
    return out[:n_sets]


# ----------------------------------------------------------------------------
# detector pixels
# ----------------------------------------------------------------------------


def bf_pixels(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Bright-field candidate pixels of the detector.

    Returns (pix, k): ``pix`` (n, 2) int detector (iy, ix); ``k`` (n, 2) the
    pixel's scattering vector (k_y, k_x) in 1/A in the scan frame:
    d = (iy - c, ix - c) * det_step, rotated by ``rotation_deg``
    (k_x = cos t d_x - sin t d_y, k_y = sin t d_x + cos t d_y), c = n_det / 2.
    Ordered by (r^2, iy, ix).
    """
    nd = w.n_det
    c = nd // 2
    iy, ix = np.mgrid[0:nd, 0:nd]
    iy = iy.ravel()
    ix = ix.ravel()
    r2 = (iy - c) ** 2 + (ix - c) ** 2
    order = np.lexsort((ix, iy, r2))
    if w.bf_nearest is not None:
        sel = order[: w.bf_nearest]
    else:
        sel = order[r2[order] <= w.bf_radius_px ** 2]
    pix = np.stack([iy[sel], ix[sel]], axis=1)
    dy = (pix[:, 0] - c).astype(np.float64) * w.optics.det_step
    dx = (pix[:, 1] - c).astype(np.float64) * w.optics.det_step
    t = math.radians(w.rotation_deg)
    kx = math.cos(t) * dx - math.sin(t) * dy
    ky = math.sin(t) * dx + math.cos(t) * dy
    return pix.astype(np.int64), np.stack([ky, kx], axis=1)


def random_weights(n: int, seed: int) -> np.ndarray:
    """Seeded per-pixel weights in [0.5, 1.5] for parity tests."""
    return np.random.default_rng(seed).uniform(0.5, 1.5, size=n)


# ----------------------------------------------------------------------------
# object contrast map and data stack
# ----------------------------------------------------------------------------


def _gaussian_filter_spectral(f: np.ndarray, sigma_px: float) -> np.ndarray:
    ny, nx = f.shape
    fy = np.fft.fftfreq(ny)[:, None]
    fx = np.fft.fftfreq(nx)[None, :]
    h = np.exp(-2.0 * (math.pi * sigma_px) ** 2 * (fy * fy + fx * fx))
    return np.real(np.fft.ifft2(np.fft.fft2(f) * h))


def object_map(n: int, step: float, sites: int, seed: int, std: float = 0.05) -> np.ndarray:
    """Seeded real contrast map on an n x n grid of pitch ``step`` (A).

    sites == 0: white noise, Gaussian-filtered (sigma 1.5 px), mean removed.
    sites > 0: a sites x sites square lattice of Gaussian blobs (sigma 0.35 A,
    weights U(0.5, 1)) mixed 0.7 / 0.3 with a filtered white background
    (sigma 10 px).  Scaled to standard deviation ``std``.
    """
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(3)[0])
    if sites == 0:
        f = _gaussian_filter_spectral(rng.standard_normal((n, n)), 1.5)
    else:
        L = n * step
        a = L / sites
        y = (np.arange(n) * step)[:, None]
        x = (np.arange(n) * step)[None, :]
        lat = np.zeros((n, n))
        wts = rng.uniform(0.5, 1.0, size=(sites, sites))
        sig = 0.35
        # periodic blobs: distance to the nearest lattice site along each axis
        for sy in range(sites):
            dy = (y - (sy + 0.5) * a + L / 2) % L - L / 2
            gy = np.exp(-dy * dy / (2 * sig * sig))
            for sx in range(sites):
                dx = (x - (sx + 0.5) * a + L / 2) % L - L / 2
                lat += wts[sy, sx] * gy * np.exp(-dx * dx / (2 * sig * sig))
        lat -= lat.mean()
        lat /= lat.std()
        bg = _gaussian_filter_spectral(rng.standard_normal((n, n)), 10.0)
        bg -= bg.mean()
        bg /= bg.std()
        f = 0.7 * lat + 0.3 * bg
    f = f - f.mean()
    return (f * (std / f.std())).astype(np.float64)


def _pixel_shifts(pix: np.ndarray, n_det: int, seed: int) -> np.ndarray:
    """Integer image shifts per pixel: a seeded linear map of the pixel offset,
    at most ~3 scan pixels at the disk edge."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(3)[2])
    c = n_det // 2
    d = (pix - c).astype(np.float64)
    rmax = max(1.0, float(np.sqrt((d * d).sum(axis=1)).max()))
    m = rng.uniform(-3.0, 3.0, size=(2, 2)) / rmax
    return np.rint(d @ m.T).astype(np.int64)


def data_stack_numpy(w: Workload, pix: np.ndarray, obj: Optional[np.ndarray] = None) -> np.ndarray:
    """G (n_bf, N, N/2+1) complex64 for small workloads, built on the CPU.

    I(r, k) = b_k (1 + 2 f(r - s_k)); with a dose, counts ~ Poisson(c I) with
    c = dose * step^2 / n_bf and I <- counts / c; G = rfft2 over the scan axes.
    """
    n = w.n_scan
    f = object_map(n, w.step, w.lattice_sites, w.seed) if obj is None else obj
    rng = np.random.default_rng(np.random.SeedSequence(w.seed).spawn(3)[2])
    nb = pix.shape[0]
    b = rng.uniform(0.95, 1.05, size=nb)
    sh = _pixel_shifts(pix, w.n_det, w.seed)
    noise = np.random.default_rng(np.random.SeedSequence(w.seed + 7).spawn(1)[0])
    cnorm = None if w.dose is None else w.dose * w.step * w.step / nb
    G = np.empty((nb, n, n // 2 + 1), dtype=np.complex64)
    for i in range(nb):
        img = b[i] * (1.0 + 2.0 * np.roll(f, (int(sh[i, 0]), int(sh[i, 1])), axis=(0, 1)))
        if cnorm is not None:
            img = noise.poisson(np.maximum(img, 0.0) * cnorm) / cnorm
        G[i] = np.fft.rfft2(img).astype(np.complex64)
    return G


def data_stack_torch(w: Workload, pix: np.ndarray, device, chunk: int = 512):
    """G (n_bf, N, N/2+1) complex64 built with plain torch ops on ``device``.

    Same recipe as :func:`data_stack_numpy` (the random stream differs: the
    Poisson draws come from a torch generator seeded with the workload seed).
    Used for the full-frame workloads, where G is ~10 GB.
    """
    import torch

    n = w.n_scan
    f = torch.as_tensor(object_map(n, w.step, w.lattice_sites, w.seed), dtype=torch.float32, device=device)
    rng = np.random.default_rng(np.random.SeedSequence(w.seed).spawn(3)[2])
    nb = pix.shape[0]
    b = torch.as_tensor(rng.uniform(0.95, 1.05, size=nb), dtype=torch.float32, device=device)
    sh = torch.as_tensor(_pixel_shifts(pix, w.n_det, w.seed), device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    cnorm = None if w.dose is None else w.dose * w.step * w.step / nb
    G = torch.empty((nb, n, n // 2 + 1), dtype=torch.complex64, device=device)
    ar = torch.arange(n, device=device)
    for s in range(0, nb, chunk):
        e = min(nb, s + chunk)
        ry = (ar[None, :] - sh[s:e, 0:1]) % n          # (c, n)
        rx = (ar[None, :] - sh[s:e, 1:2]) % n
        img = f[ry[:, :, None], rx[:, None, :]]          # (c, n, n)
        img = b[s:e, None, None] * (1.0 + 2.0 * img)
        if cnorm is not None:
            img = torch.poisson(torch.clamp(img, min=0.0) * cnorm, generator=gen) / cnorm
        G[s:e] = torch.fft.rfft2(img)
        del img
    return G
