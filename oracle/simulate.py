"""Physical forward models used by the oracle's own pins.

TEST INFRASTRUCTURE ONLY (see the package docstring).

``first_order_G`` writes the weak-object data model directly from the probe
amplitude A(k) = a(k) exp(-i chi(k)); ``wave_optics_G`` is a brute-force
simulation (shifted probe times object, far-field intensity, Fourier transform
over probe positions) that pins the first-order model, and with it the sign,
lobe, alias and tilt conventions of the transfer.

Derivation of the first-order model (numpy's exp(-2 pi i) forward
convention).  With object transmission 1 + c(r), c = A_l + i phi,
c(r) = sum_K c^(K) exp(2 pi i K.r), the far field of the probe at r_p is
Psi(k) = A(k) e^{-2 pi i k.r_p} + sum_K c^(K) A(k - K) e^{-2 pi i (k-K).r_p}.
To first order in c, |Psi|^2 = a(k)^2 + sum_K c^(K) conj A(k) A(k-K)
e^{2 pi i K.r_p} + c.c., and summing over the N x N probe positions with
exp(-2 pi i q.r_p) keeps the fine frequencies K = q (mod N dq):
    G(q, k) = N^2 a(k)^2 [q = 0]
            + N^2 sum_{K = q} [ c^(K) conj A(k) A(k - K)
                               + conj(c^(-K)) A(k) conj A(k + K) ].
With c sampled on the u N fine grid, N^2 c^(K) = fft2(c)[K] / u^2.

The probe here is written from the physics on its own, sharing nothing with
the oracle's aperture and aberration functions, so the simulation pins them
too: the objective aperture is a disc of semi-angle alpha (a hard stop, or a
stop whose transmission falls linearly to zero over one detector pixel
centred on the edge, the antialiased stop of "Tilt-corrected SSB on CUDA"
Changes), and the aberration phase is the Krivanek series written with the
complex beam angle w = theta_x + i theta_y, in which the term C_nm of radial
order n and azimuthal order m is |w|^(n+1-m) Re[w^m e^(-i m phi_nm)] /
(n + 1), times 2 pi / lambda.
"""
from __future__ import annotations

import math

import numpy as np


def _signed(i, n: int):
    """Signed frequency index of stored row i of an n-point FFT axis."""
    i = np.asarray(i)
    return np.where(i < n // 2, i, i - n)


def objective_aperture(ky, kx, optics):
    """Transmission of the objective stop at scattering vector k (1/A): the
    beam angle lambda |k| against the semi-angle alpha.  Hard stop: 1 inside
    the disc, its rim included, 0 outside.  Antialiased stop: the
    transmission falls linearly from 1 to 0 across one detector pixel dk
    centred on the rim, 1 - (|k| - alpha/lambda + dk/2) / dk clipped to
    [0, 1]."""
    r = np.hypot(np.asarray(ky, dtype=np.float64), np.asarray(kx, dtype=np.float64))
    rim = optics.semiangle / optics.wavelength
    if not optics.soft:
        return np.where(r <= rim, 1.0, 0.0)
    return np.minimum(1.0, np.maximum(0.0, 1.0 - (r - rim + 0.5 * optics.det_step) / optics.det_step))


def aberration_phase(ky, kx, optics):
    """Aberration phase (rad) of the beam at scattering vector k: with the
    complex beam angle w = theta_x + i theta_y, theta = lambda k + tilt,
    chi = (2 pi / lambda) sum_nm C_nm |w|^(n+1-m) Re[w^m e^(-i m phi_nm)] / (n+1)."""
    lam = optics.wavelength
    w = (lam * np.asarray(kx, dtype=np.float64) + optics.tilt[1]) + 1j * (
        lam * np.asarray(ky, dtype=np.float64) + optics.tilt[0])
    aw = np.abs(w)
    acc = np.zeros(w.shape, dtype=np.float64)
    for (n, m, c, phi) in optics.aberrations:
        acc = acc + c * aw ** (n + 1 - m) * np.real(w ** m * np.exp(-1j * m * phi)) / (n + 1)
    return acc * (2.0 * math.pi / lam)


def probe_amplitude(ky, kx, optics):
    """Probe wave in the far field, A(k) = aperture(k) exp(-i chi(k))."""
    return objective_aperture(ky, kx, optics) * np.exp(-1j * aberration_phase(ky, kx, optics))


def fine_spectrum(field: np.ndarray, upsampling: int) -> np.ndarray:
    """fft2(field) / u^2 of a (uN, uN) fine-grid field: the object-spectrum
    value the data model multiplies at each fine frequency."""
    return np.fft.fft2(field) / float(upsampling * upsampling)


def first_order_G(k: np.ndarray, c_fine: np.ndarray, n_scan: int, step: float, upsampling: int,
                  optics, include_dc: bool = True) -> np.ndarray:
    """Noise-free first-order data (n_bf, N, N/2+1) complex128 for the complex
    fine-grid object c = A_l + i phi (module docstring).  Every fine alias of
    every stored frequency is summed (no alias rule applied)."""
    n = n_scan
    nf = upsampling * n
    dq = 1.0 / (n * step)
    F = np.fft.fft2(c_fine) / float(upsampling * upsampling)
    ky, kx = k[:, 0], k[:, 1]
    A0 = probe_amplitude(ky, kx, optics)
    G = np.zeros((k.shape[0], n, n // 2 + 1), dtype=np.complex128)
    half = nf // 2
    for iy in range(n):
        yh = int(_signed(iy, n))
        for ix in range(n // 2 + 1):
            acc = np.zeros(k.shape[0], dtype=np.complex128)
            for jy in range(-upsampling, upsampling + 1):
                Ky = yh + jy * n
                if Ky < -half or Ky >= half:
                    continue
                for jx in range(-upsampling, upsampling + 1):
                    Kx = ix + jx * n
                    if Kx < -half or Kx >= half:
                        continue
                    cK = F[Ky % nf, Kx % nf]
                    cmK = F[(-Ky) % nf, (-Kx) % nf]
                    Qy, Qx = Ky * dq, Kx * dq
                    Am = probe_amplitude(ky - Qy, kx - Qx, optics)
                    Ap = probe_amplitude(ky + Qy, kx + Qx, optics)
                    acc += cK * np.conj(A0) * Am + np.conj(cmK) * A0 * np.conj(Ap)
            G[:, iy, ix] = acc          # F already holds N^2 c^(K) = fft2(c)[K] / u^2
            if include_dc and iy == 0 and ix == 0:
                G[:, iy, ix] += n * n * np.abs(A0) ** 2
    return G


def band_limited_field(nf: int, rng: np.random.Generator, std: float = 1.0, cutoff: float = 1.0) -> np.ndarray:
    """Real seeded field on an nf x nf grid whose spectrum is zero on the
    Nyquist lines and beyond ``cutoff`` x Nyquist (so Fourier interpolation to
    a finer grid is exact)."""
    f = rng.standard_normal((nf, nf))
    F = np.fft.fft2(f)
    fy = np.fft.fftfreq(nf)[:, None] * nf
    fx = np.fft.fftfreq(nf)[None, :] * nf
    keep = (np.abs(fy) < nf // 2) & (np.abs(fx) < nf // 2) & (np.hypot(fy, fx) <= cutoff * nf / 2)
    keep[0, 0] = False
    f = np.real(np.fft.ifft2(F * keep))
    return f * (std / f.std())


def wave_optics_G(n_scan: int, step: float, m_sim: int, optics, c_fine: np.ndarray, upsampling: int,
                  n_slices: int = 1):
    """Brute-force data for object transmission exp(c), c = A_l + i phi.

    The simulation grid spans the scan's field of view L = N s with m_sim
    pixels per axis (pitch L / m_sim); its far-field pixels are the scan
    frequencies themselves (spacing dq = 1/L), which serve as the detector.
    The probe is ifft2(A(k)), shifted by whole simulation pixels to each of
    the N x N scan positions; the object is the fine-grid field Fourier
    interpolated onto the simulation grid.  Returns (k (m^2, 2) detector
    vectors (1/A), G (m^2, N, N/2+1) complex128).

    With optics.depth = t > 0 the object is a multislice stack: n_slices
    slices of transmission exp(c / n_slices) at depths (j + 1/2) t /
    n_slices below the plane chi refers to, the wave propagated between them
    by the paraxial Fresnel factor exp(-i pi dz |lambda k + tau|^2 / lambda)
    (beam direction theta = lambda k + tau, numpy's exp(+2 pi i k.r) inverse
    transform).  The far-field intensity after the last slice is the data.
    """
    n = n_scan
    m = m_sim
    nf = upsampling * n
    assert m % n == 0 and m >= 2 * nf
    shift = m // n
    L = n * step
    f = np.fft.fftfreq(m, d=L / m)
    KY, KX = np.meshgrid(f, f, indexing="ij")
    psi = np.fft.ifft2(probe_amplitude(KY, KX, optics))
    F = np.fft.fft2(c_fine)
    Fs = np.zeros((m, m), dtype=np.complex128)
    idx = _signed(np.arange(nf), nf)
    Fs[np.ix_(idx % m, idx % m)] = F
    c_sim = np.fft.ifft2(Fs) * (m / nf) ** 2
    t = float(getattr(optics, "depth", 0.0))
    I = np.empty((n, n, m, m))
    if t == 0.0:
        obj = np.exp(c_sim)
        for py in range(n):
            for px in range(n):
                ps = np.roll(psi, (py * shift, px * shift), axis=(0, 1))
                I[py, px] = np.abs(np.fft.fft2(ps * obj)) ** 2
    else:
        lam = optics.wavelength
        th2 = (lam * KY + optics.tilt[0]) ** 2 + (lam * KX + optics.tilt[1]) ** 2
        dz = t / n_slices

        def prop(z):
            return np.exp(-1j * math.pi * z * th2 / lam)

        first, between = prop(0.5 * dz), prop(dz)
        sl = np.exp(c_sim / n_slices)
        for py in range(n):
            for px in range(n):
                ps = np.roll(psi, (py * shift, px * shift), axis=(0, 1))
                W = np.fft.fft2(ps) * first
                for j in range(n_slices):
                    if j:
                        W = W * between
                    W = np.fft.fft2(np.fft.ifft2(W) * sl)
                I[py, px] = np.abs(W) ** 2
    G = np.fft.rfft2(I, axes=(0, 1))                    # (n, n/2+1, m, m)
    G = np.transpose(G, (2, 3, 0, 1)).reshape(m * m, n, n // 2 + 1)
    k = np.stack([KY.ravel(), KX.ravel()], axis=1)
    return k, G
