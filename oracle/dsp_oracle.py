"""Plain FP64 oracle of the regularized direct-ptychography hot path.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and obviously
correct: every function evaluates the definition it cites with NumPy in
float64 / complex128, vectorized over bright-field pixels and looped over
scan frequencies.  No blocking, fusion or reordering beyond that.

Pages:
  [P1]  "Where the 9 s of regularized preparation goes" (Code path; Raw
        numbers) and its later section "Preparation in one kernel per alias
        count: 9.1 s to 35 ms" (What changed).
  [P3]  "Tilt-corrected SSB on CUDA: fit and preview speed" (Setup; Changes).
  [P4]  "Historical WebGPU G(q,k) memory experiment" (Why herm is exactly
        lossless; Implementation; Object-redraw fast path).

Readings where the pages are silent are the ones listed in the design notes
(frequency set, alias rule, aperture edge, aberration convention, tilt,
weights, scale, prior, agreement); each function states the one it uses.

Parity unpinned (values fixed by these readings, not by the pages): the
strength scale (sum of weights), the prior's constant s_p, the weights, the
agreement's normalisation, the rotation sign, the previews' correction (the
SSB sum's matched filter conj(Gamma)) and the loss (the weighted mean
variance of the pixels' phases).
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# frequencies and aliases
# ----------------------------------------------------------------------------


def signed_index(i, n: int):
    """Signed FFT index of stored row i of an n-point axis: i for i < n/2,
    else i - n."""
    i = np.asarray(i)
    return np.where(i < n // 2, i, i - n)


def scan_frequency_step(n_scan: int, step: float) -> float:
    """dq = 1 / (N s): spacing of the scan-frequency grid (1/A)."""
    return 1.0 / (n_scan * step)


def unique_frequencies(n_scan: int) -> np.ndarray:
    """Scan frequencies solved by the prepare, as stored (iy, ix), row-major.

    [P1] Code path: 130560 frequencies at a 512 x 512 scan.  Reading: the
    Hermitian half plane (ix in [0, N/2]) without the Nyquist column
    (ix = N/2), without the Nyquist row (iy = N/2), and without the column
    ix = 0 for signed row <= 0 (DC, and the conjugates of ix = 0 entries with
    signed row > 0).  |U| = N (N - 2) / 2.
    """
    n = n_scan
    out = []
    for iy in range(n):
        if iy == n // 2:
            continue
        yh = iy if iy < n // 2 else iy - n
        for ix in range(n // 2):
            if ix == 0 and yh <= 0:
                continue
            out.append((iy, ix))
    return np.asarray(out, dtype=np.int64).reshape(-1, 2)


def alias_radius(optics) -> float:
    """Largest |Q| at which the two aperture supports still overlap.

    Soft aperture: support radius alpha/lambda + dk/2 each, so
    R = 2 alpha / lambda + dk.  Hard aperture: R = 2 alpha / lambda.
    ([P1] Raw numbers' alias-count histogram is reproduced exactly by this R.)
    """
    r = (2.0 * optics.semiangle) / optics.wavelength
    if optics.soft:
        r = r + optics.det_step
    return r


def aliases_of(iy: int, ix: int, n_scan: int, upsampling: int, dq: float, R: float) -> List[Tuple[int, int]]:
    """Fine-grid aliases K of the stored frequency (iy, ix) that carry signal.

    The upsampled grid has u N points per axis, indices in [-uN/2, uN/2).
    K = (yh + j_y N, ix + j_x N) for integers j; K is kept when
    |K|^2 dq^2 < R^2 (the two apertures overlap).  Order: (j_y, j_x)
    ascending.  [P1] Code path (frequencies bucketed by alias count).
    """
    n = n_scan
    half = (upsampling * n) // 2
    yh = iy if iy < n // 2 else iy - n
    out = []
    for jy in range(-upsampling, upsampling + 1):
        ky = yh + jy * n
        if ky < -half or ky >= half:
            continue
        for jx in range(-upsampling, upsampling + 1):
            kx = ix + jx * n
            if kx < -half or kx >= half:
                continue
            k2 = float(ky * ky + kx * kx)
            if k2 * (dq * dq) < R * R:
                out.append((ky, kx))
    return out


def alias_table(n_scan: int, step: float, upsampling: int, optics):
    """(q (n_q, 2) stored indices, counts (n_q,), K list of (A_q, 2) arrays)."""
    q = unique_frequencies(n_scan)
    dq = scan_frequency_step(n_scan, step)
    R = alias_radius(optics)
    Ks = [np.asarray(aliases_of(int(a), int(b), n_scan, upsampling, dq, R), dtype=np.int64).reshape(-1, 2)
          for a, b in q]
    counts = np.asarray([k.shape[0] for k in Ks], dtype=np.int64)
    return q, counts, Ks


def alias_histogram(counts: np.ndarray) -> Dict[int, int]:
    vals, num = np.unique(counts, return_counts=True)
    return {int(v): int(c) for v, c in zip(vals, num)}


# ----------------------------------------------------------------------------
# probe optics
# ----------------------------------------------------------------------------


def aperture(kabs, optics):
    """Aperture amplitude a(|k|) (real).

    Soft ([P3] Changes, Geometry: the edge's denominator is the constant
    detector step): a = clip(1/2 + (alpha/lambda - |k|) / dk, 0, 1), a linear
    ramp one detector pixel wide centred on the aperture radius.
    Hard: a = 1 for |k| <= alpha/lambda, else 0.
    """
    kabs = np.asarray(kabs, dtype=np.float64)
    kc = optics.semiangle / optics.wavelength
    if optics.soft:
        return np.clip(0.5 + (kc - kabs) / optics.det_step, 0.0, 1.0)
    return (kabs <= kc).astype(np.float64)


def active_pixels(k: np.ndarray, optics) -> np.ndarray:
    """Indices of candidate pixels with non-zero aperture weight, in input
    order ([P4] gotchas: the active set, not the labelled set, carries G)."""
    a = aperture(np.hypot(k[:, 0], k[:, 1]), optics)
    return np.nonzero(a > 0.0)[0]


def chi(ky, kx, optics):
    """Aberration phase chi(k) (rad) in Krivanek polar notation.

    theta = lambda k + tau (tilt shifts the angle at which chi is evaluated),
    |theta| = t, azimuth p = atan2(theta_y, theta_x):
        chi = (2 pi / lambda) sum_nm C_nm t^(n+1) / (n+1) cos(m (p - phi_nm)).
    [P1] Setup: the fit holds 14 aberration terms (radial orders 1..5) and a
    tilt.  Probe amplitude A(k) = a(k) exp(-i chi(k)).
    """
    lam = optics.wavelength
    ty = lam * np.asarray(ky, dtype=np.float64) + optics.tilt[0]
    tx = lam * np.asarray(kx, dtype=np.float64) + optics.tilt[1]
    t = np.hypot(ty, tx)
    p = np.arctan2(ty, tx)
    acc = np.zeros(np.broadcast(ty, tx).shape)
    for (n, m, c, phi) in optics.aberrations:
        acc = acc + c * t ** (n + 1) / (n + 1) * np.cos(m * (p - phi))
    return (2.0 * math.pi / lam) * acc


def depth_factor(delta, optics):
    """Depth term of one lobe for a weak object spread evenly through the
    thickness t = optics.depth (A) downstream of the plane chi refers to.

    A slice at depth z sees the probe propagated by z, A(k) exp(-i pi z
    |theta_k|^2 / lambda) (paraxial, theta_k = lambda k + tau the beam
    direction, so a tilted beam also walks sideways with depth).  The lobe
    built from the probe at k and at k' then carries exp(i pi z delta /
    lambda) with delta = |theta_k|^2 - |theta_k'|^2 (L) or |theta_k'|^2 -
    |theta_k|^2 (R); its mean over z in [0, t] is
        exp(i phi / 2) sinc(phi / 2),   phi = pi t delta / lambda,
    the "sinc and phase factor" of [P1] What changed 2 and of the thick-sample
    fits of [P3] Where the time went.  Exactly 1 at t = 0.
    """
    t = float(getattr(optics, "depth", 0.0))
    delta = np.asarray(delta, dtype=np.float64)
    if t == 0.0:
        return np.ones(delta.shape, dtype=np.complex128)
    h = 0.5 * math.pi * t * delta / optics.wavelength
    return np.exp(1j * h) * np.sinc(h / math.pi)          # np.sinc(x) = sin(pi x) / (pi x)


def lobes(ky, kx, Qy: float, Qx: float, optics):
    """The two weak-object lobes at scattering vector k for object frequency Q.

    L = a(k) a(k - Q) exp(+i [chi(k) - chi(k - Q)])      (= conj A(k) A(k - Q))
    R = a(k) a(k + Q) exp(-i [chi(k) - chi(k + Q)])      (= A(k) conj A(k + Q))
    Each is exactly zero where its two apertures do not overlap ([P1] What
    changed 2: exact zeros skipped).  With a depth, each lobe is multiplied by
    its depth_factor (1 at depth 0).
    """
    ky = np.asarray(ky, dtype=np.float64)
    kx = np.asarray(kx, dtype=np.float64)
    a0 = aperture(np.hypot(ky, kx), optics)
    am = aperture(np.hypot(ky - Qy, kx - Qx), optics)
    ap = aperture(np.hypot(ky + Qy, kx + Qx), optics)
    c0 = chi(ky, kx, optics)
    cm = chi(ky - Qy, kx - Qx, optics)
    cp = chi(ky + Qy, kx + Qx, optics)
    L = a0 * am * np.exp(1j * (c0 - cm))
    R = a0 * ap * np.exp(-1j * (c0 - cp))
    if float(getattr(optics, "depth", 0.0)) != 0.0:
        lam = optics.wavelength
        ty, tx = optics.tilt

        def th2(y, x):
            return (lam * y + ty) ** 2 + (lam * x + tx) ** 2

        t0 = th2(ky, kx)
        L = L * depth_factor(t0 - th2(ky - Qy, kx - Qx), optics)
        R = R * depth_factor(th2(ky + Qy, kx + Qx) - t0, optics)
    return L, R


def transfer(k: np.ndarray, Q: np.ndarray, optics, method: str) -> np.ndarray:
    """Transfer matrix T (n_k, d) of one scan frequency.

    For object c = A_l + i phi (log-amplitude, phase) the first-order data is
    G = sum_Q [T_A(Q) A_l(Q) + T_phi(Q) phi(Q)] with T_A = L + R and
    T_phi = i (L - R).  Columns: phase method [T_phi(Q_1..Q_A)];
    complex method [T_A(Q_1..Q_A), T_phi(Q_1..Q_A)] ([P1] conclusion 3: the
    phase system is the complex system's lower-right block).
    """
    cols_a, cols_p = [], []
    for Qy, Qx in Q:
        L, R = lobes(k[:, 0], k[:, 1], float(Qy), float(Qx), optics)
        cols_a.append(L + R)
        cols_p.append(1j * (L - R))
    if method == "phase":
        cols = cols_p
    elif method == "complex":
        cols = cols_a + cols_p
    else:
        raise ValueError(method)
    if not cols:
        return np.zeros((k.shape[0], 0), dtype=np.complex128)
    return np.stack(cols, axis=1)


# ----------------------------------------------------------------------------
# normal equations, prior, eigenbasis, solves
# ----------------------------------------------------------------------------


def normal_equations(T: np.ndarray, g: np.ndarray, w: np.ndarray):
    """M = T^H W T, r = T^H W g, P = g^H W g with W = diag(w) ([P1] Code path:
    Gram and right side per frequency; signal power)."""
    g = np.asarray(g, dtype=np.complex128)
    wT = w[:, None] * T
    M = T.conj().T @ wT
    r = T.conj().T @ (w * g)
    P = float(np.sum(w * (g.real * g.real + g.imag * g.imag)))
    return M, r, P


def prior(Q_invA: np.ndarray, smoothness: float) -> np.ndarray:
    """Per-unknown Tikhonov weight p = (1 + |Q|^2 / s^2)^2 ([P1] Raw numbers:
    the prior stage); p = 1 when s <= 0."""
    if smoothness <= 0:
        return np.ones(Q_invA.shape[0])
    q2 = Q_invA[:, 0] ** 2 + Q_invA[:, 1] ** 2
    return (1.0 + q2 / (smoothness * smoothness)) ** 2


def phase_eigenbasis(M: np.ndarray, r: np.ndarray, p: np.ndarray):
    """Eigenbasis that makes every strength a diagonal evaluation ([P1] Code
    path: batched eigh for phase).

    C = D^-1/2 M D^-1/2 = V diag(lam) V^H (lam ascending), D = diag(p);
    U = D^-1/2 V; c = V^H D^-1/2 r.  Then (M + mu D)^-1 r = U (c / (lam + mu)).
    """
    s = 1.0 / np.sqrt(p)
    C = M * s[:, None] * s[None, :]
    lam, V = np.linalg.eigh(C)
    U = V * s[:, None]
    c = V.conj().T @ (s * r)
    return lam, U, c


def solve_phase(lam: np.ndarray, U: np.ndarray, c: np.ndarray, mu: float) -> np.ndarray:
    """x = U (c / (lam + mu)), mu = strength * scale."""
    return U @ (c / (lam + mu))


def solve_direct(M: np.ndarray, r: np.ndarray, reg_diag: np.ndarray) -> np.ndarray:
    """x = (M + diag(reg_diag))^-1 r, the regularized normal equations."""
    return np.linalg.solve(M + np.diag(reg_diag.astype(np.complex128)), r)


def residual(M: np.ndarray, r: np.ndarray, P: float, x: np.ndarray) -> float:
    """Weighted data misfit sum_k w |g - T x|^2 = P - 2 Re(x^H r) + x^H M x."""
    return float(P - 2.0 * np.real(np.vdot(x, r)) + np.real(np.vdot(x, M @ x)))


def strength_scale(w_active: np.ndarray) -> float:
    """Strength unit: the sum of the active pixels' weights, so a strength is a
    fraction of the data term's scale ([P1] Rejected ideas mention strengths
    down to 0.01 of the scale)."""
    return float(np.sum(w_active))


# ----------------------------------------------------------------------------
# prepare / solve over many frequencies
# ----------------------------------------------------------------------------


class Prepared:
    """Per-frequency systems for a list of frequencies (oracle side).

    Attributes (lists over the frequencies, compact per frequency):
      q (n, 2) stored indices; K list of (A, 2) alias indices; A (n,);
      M, r, P, p; for phase: lam, U, c.  scale is the strength unit.
    """

    def __init__(self):
        self.q = None
        self.K = []
        self.A = None
        self.M, self.r, self.P, self.p = [], [], [], []
        self.lam, self.U, self.c = [], [], []
        self.scale = 0.0
        self.method = "phase"


def prepare(q_list: np.ndarray, gcols: Sequence[np.ndarray], k_act: np.ndarray, w_act: np.ndarray,
            n_scan: int, step: float, upsampling: int, optics, method: str, smoothness: float) -> Prepared:
    """Prepare the regularized systems of the frequencies ``q_list``.

    gcols[i] holds G(q_i, k) over the active pixels (k_act, w_act).  Follows
    [P1] Code path: aliases per frequency, prior, gather G, transfer,
    Gram T^H W T, right side T^H W g, signal power, then (phase) the
    eigendecomposition and projection.
    """
    dq = scan_frequency_step(n_scan, step)
    R = alias_radius(optics)
    out = Prepared()
    out.method = method
    out.q = np.asarray(q_list, dtype=np.int64).reshape(-1, 2)
    out.scale = strength_scale(w_act)
    A = []
    for i, (iy, ix) in enumerate(out.q):
        K = np.asarray(aliases_of(int(iy), int(ix), n_scan, upsampling, dq, R), dtype=np.int64).reshape(-1, 2)
        Q = K.astype(np.float64) * dq
        T = transfer(k_act, Q, optics, method)
        M, r, P = normal_equations(T, gcols[i], w_act)
        p1 = prior(Q, smoothness)
        p = np.concatenate([p1, p1]) if method == "complex" else p1
        out.K.append(K)
        A.append(K.shape[0])
        out.M.append(M)
        out.r.append(r)
        out.P.append(P)
        out.p.append(p)
        if method == "phase":
            lam, U, c = phase_eigenbasis(M, r, p)
            out.lam.append(lam)
            out.U.append(U)
            out.c.append(c)
    out.A = np.asarray(A, dtype=np.int64)
    return out


def solve(prep: Prepared, strength, use_eigenbasis: bool = True) -> List[np.ndarray]:
    """Solutions x (compact, per frequency) at one strength.

    phase: strength is a float lambda; x = U (c / (lam + lambda scale)) or,
    with use_eigenbasis False, the direct solve of (M + lambda scale D) x = r.
    complex: strength is (lambda_A, lambda_phi); x = (M + scale diag(lambda_A p,
    lambda_phi p))^-1 r, x = [A_l(Q_1..Q_A), phi(Q_1..Q_A)].
    """
    out = []
    for i in range(len(prep.M)):
        A = int(prep.A[i])
        if prep.method == "phase":
            mu = float(strength) * prep.scale
            if use_eigenbasis:
                x = solve_phase(prep.lam[i], prep.U[i], prep.c[i], mu)
            else:
                x = solve_direct(prep.M[i], prep.r[i], mu * prep.p[i])
        else:
            la, lp = strength
            reg = prep.scale * np.concatenate([la * prep.p[i][:A], lp * prep.p[i][A:]])
            x = solve_direct(prep.M[i], prep.r[i], reg)
        out.append(x)
    return out


def scatter(q_list: np.ndarray, Ks: Sequence[np.ndarray], xs: Sequence[np.ndarray], n_scan: int,
            upsampling: int, n_comp: int) -> np.ndarray:
    """Place packed solutions on the fine half plane (n_comp, uN, uN/2+1).

    Alias K = (K_y, K_x) goes to (K_y mod uN, K_x) when K_x > 0 or
    (K_x = 0 and K_y >= 0); otherwise its conjugate goes to (-K)
    ([P4] Why herm is exactly lossless: a real field's spectrum at -q is the
    conjugate of the one at q).  Entries never reached stay 0.
    """
    nf = upsampling * n_scan
    out = np.zeros((n_comp, nf, nf // 2 + 1), dtype=np.complex128)
    for K, x in zip(Ks, xs):
        A = K.shape[0]
        for c in range(n_comp):
            for m in range(A):
                v = x[c * A + m]
                ky, kx = int(K[m, 0]), int(K[m, 1])
                if kx > 0 or (kx == 0 and ky >= 0):
                    out[c, ky % nf, kx] = v
                else:
                    out[c, (-ky) % nf, -kx] = np.conj(v)
    return out


# ----------------------------------------------------------------------------
# SSB / agreement streaming sum
# ----------------------------------------------------------------------------


def stored_frequencies(n_scan: int, step: float) -> np.ndarray:
    """|q| (N, N/2+1) of every stored half-plane entry (1/A)."""
    dq = scan_frequency_step(n_scan, step)
    iy = signed_index(np.arange(n_scan), n_scan).astype(np.float64)[:, None]
    ix = np.arange(n_scan // 2 + 1, dtype=np.float64)[None, :]
    return np.hypot(iy * dq, ix * dq)


def band_mask(n_scan: int, step: float, band: Optional[Tuple[float, float]]) -> np.ndarray:
    """Stored entries with f_lo <= |q| <= f_hi ([P3] Setup: the 0.2 to 0.9 1/A
    fit band holds 44,247 frequencies at the 512 x 512 scan)."""
    f = stored_frequencies(n_scan, step)
    if band is None:
        return np.ones_like(f, dtype=bool)
    return (f >= band[0]) & (f <= band[1])


def ssb_entry(k_act: np.ndarray, w_act: np.ndarray, g: np.ndarray, qy: float, qx: float, optics):
    """SSB sums at one stored frequency q (no aliases):
    Gamma = T_phi(q, k) = i (L - R);  S = sum_k w conj(Gamma) g;
    N = sum_k w |Gamma|^2.  ([P4] Object-redraw fast path: sum the corrected
    G over bright-field pixels in Fourier space.)"""
    L, R = lobes(k_act[:, 0], k_act[:, 1], qy, qx, optics)
    gam = 1j * (L - R)
    S = np.sum(w_act * np.conj(gam) * np.asarray(g, dtype=np.complex128))
    Nn = float(np.sum(w_act * (gam.real ** 2 + gam.imag ** 2)))
    return complex(S), Nn


def ssb(entries: np.ndarray, gcols: Sequence[np.ndarray], k_act: np.ndarray, w_act: np.ndarray,
        n_scan: int, step: float, sets: Sequence):
    """S (B, n), N (B, n) at the stored entries ``entries`` (n, 2) for each
    optics set.  gcols[i] = G(entry i, active k)."""
    dq = scan_frequency_step(n_scan, step)
    B = len(sets)
    S = np.zeros((B, len(entries)), dtype=np.complex128)
    Nn = np.zeros((B, len(entries)))
    for i, (iy, ix) in enumerate(entries):
        qy = float(signed_index(int(iy), n_scan)) * dq
        qx = float(ix) * dq
        for b in range(B):
            S[b, i], Nn[b, i] = ssb_entry(k_act, w_act, gcols[i], qy, qx, sets[b])
    return S, Nn


def agreement(S: np.ndarray, Nn: np.ndarray, power: np.ndarray) -> np.ndarray:
    """Fraction of the band's weighted signal power the SSB model explains:
    E = sum_{band, N > 0} |S|^2 / N  /  sum_{band} sum_k w |g|^2.
    (Variable projection of the one-parameter-per-frequency fit; [P3] Where
    the time went: one agreement pass evaluates several parameter sets.)"""
    num = np.zeros(S.shape[0])
    for b in range(S.shape[0]):
        m = Nn[b] > 0
        num[b] = np.sum((S[b, m].real ** 2 + S[b, m].imag ** 2) / Nn[b, m])
    return num / float(np.sum(power))


# ----------------------------------------------------------------------------
# previews and the loss path
# ----------------------------------------------------------------------------


def g_full(G_act: np.ndarray, iy: int, ix: int, n_scan: int) -> np.ndarray:
    """G(q, k) over the given pixels at any full-plane index (iy, ix) from the
    stored half plane: G(-q, k) = conj G(q, k) ([P4] Why herm is exactly
    lossless)."""
    iy %= n_scan
    ix %= n_scan
    if ix <= n_scan // 2:
        return np.asarray(G_act[:, iy, ix], dtype=np.complex128)
    return np.conj(np.asarray(G_act[:, (-iy) % n_scan, n_scan - ix], dtype=np.complex128))


def corrected_term(ka: np.ndarray, wa: np.ndarray, G_act: np.ndarray, Ky: int, Kx: int, n_scan: int,
                   step: float, optics) -> np.ndarray:
    """Per-pixel corrected G at fine frequency K (signed indices), K != 0:
    C_k(K) = i w_k conj(Gamma(K, k)) G(K mod N, k) with Gamma = T_phi = i (L - R)
    at Q = K dq.  ([P4] Object-redraw fast path: the gamma-corrected G(q, k);
    [P3] Open: the corrected spectrum of a real image is anti-Hermitian except
    at DC, which the factor i gives.)  Reading, parity unpinned as a
    definition: the correction is the SSB sum's matched filter conj(Gamma)."""
    dq = scan_frequency_step(n_scan, step)
    L, R = lobes(ka[:, 0], ka[:, 1], Ky * dq, Kx * dq, optics)
    gam = 1j * (L - R)
    return 1j * wa * np.conj(gam) * g_full(G_act, Ky, Kx, n_scan)


def preview_spectrum(G: np.ndarray, k: np.ndarray, w: Optional[np.ndarray], n_scan: int, step: float,
                     upsampling: int, optics) -> np.ndarray:
    """Fine half plane P (uN, uN/2 + 1) of the object fast path: the corrected
    G summed over the active pixels at every fine frequency K (signed row,
    column 0..uN/2), P(K) = sum_k C_k(K); at K = 0 the uncorrected
    P(0) = sum_k w_k G(0, k).  ([P4] Object-redraw fast path: sum over BF
    pixels in Fourier space, then one inverse FFT; [P3] Changes: the 1x and
    3x drag previews.)  The fine grid's Nyquist row and column stay 0: index
    uN/2 stands for two frequencies, +-uN/2 dq, whose corrections differ, so
    no anti-Hermitian value exists there (the reading the prepare takes for
    the Nyquist lines' aliases)."""
    act = active_pixels(k, optics)
    ka = k[act]
    wa = np.ones(len(act)) if w is None else np.asarray(w, dtype=np.float64)[act]
    Ga = G[act]
    m = upsampling * n_scan
    P = np.zeros((m, m // 2 + 1), dtype=np.complex128)
    for iy in range(m):
        Ky = int(signed_index(iy, m))
        for Kx in range(m // 2 + 1):
            if Ky == -(m // 2) or Kx == m // 2:
                continue
            if Ky == 0 and Kx == 0:
                P[0, 0] = np.sum(wa * np.asarray(Ga[:, 0, 0], dtype=np.complex128))
            else:
                P[iy, Kx] = np.sum(corrected_term(ka, wa, Ga, Ky, Kx, n_scan, step, optics))
    return P


def full_plane(P: np.ndarray) -> np.ndarray:
    """The (M, M) plane from its half (M, M/2 + 1) by P(-K) = -conj P(K) for
    K != 0 ([P3] Open: anti-Hermitian except at DC)."""
    m = P.shape[0]
    F = np.zeros((m, m), dtype=np.complex128)
    F[:, : m // 2 + 1] = P
    for iy in range(m):
        for ix in range(m // 2 + 1, m):
            F[iy, ix] = -np.conj(P[(-iy) % m, m - ix])
    return F


def preview_phase(P: np.ndarray) -> np.ndarray:
    """Object phase of the fast path, angle(ifft2(full plane)) on the (M, M)
    grid ([P4] Object-redraw fast path: ONE 2D inverse FFT and one atan2;
    the estimator angle(mean(object)))."""
    return np.angle(np.fft.ifft2(full_plane(P)))


def pixel_planes(G: np.ndarray, k: np.ndarray, w: Optional[np.ndarray], n_scan: int, step: float, optics):
    """Yields (w_k, C_k) for every active pixel: its corrected full (N, N)
    plane, the corrected terms at every q != 0 and w_k G(0, k) at DC ([P3]
    Changes, loss path: the corrected full plane straight from the stored
    half plane).  The Nyquist row and column are 0, as in the preview
    (index N/2 stands for +-N/2 dq)."""
    act = active_pixels(k, optics)
    ka = k[act]
    wa = np.ones(len(act)) if w is None else np.asarray(w, dtype=np.float64)[act]
    Ga = G[act]
    n = n_scan
    dq = scan_frequency_step(n, step)
    yy = signed_index(np.arange(n), n).astype(np.float64)
    QY, QX = np.meshgrid(yy * dq, yy * dq, indexing="ij")     # full-plane signed frequencies
    iy = np.arange(n)[:, None]
    ix = np.arange(n)[None, :]
    direct = np.broadcast_to(ix <= n // 2, (n, n))
    src_y = np.where(direct, iy, (-iy) % n)       # G(-q) = conj G(q) beyond column N/2
    src_x = np.where(direct, ix, n - ix)
    for j in range(len(act)):
        gfull = np.asarray(Ga[j], dtype=np.complex128)[src_y, src_x]
        gfull = np.where(direct, gfull, np.conj(gfull))
        L, R = lobes(np.full(QY.shape, ka[j, 0]), np.full(QY.shape, ka[j, 1]), QY, QX, optics)
        C = 1j * wa[j] * np.conj(1j * (L - R)) * gfull
        C[0, 0] = wa[j] * gfull[0, 0]
        C[n // 2, :] = 0.0
        C[:, n // 2] = 0.0
        yield float(wa[j]), C


def loss_path(G: np.ndarray, k: np.ndarray, w: Optional[np.ndarray], n_scan: int, step: float, optics):
    """Mean phase and loss over the pixels' objects ([P3] Changes, loss path:
    inverse FFT of each pixel's corrected plane and phase moments; [P4]:
    mean(angle(object)) needs the per-pixel phases).  Pixel k's object is
    o_k = ifft2(C_k), theta_k = angle(o_k).  Returns (mean phase
    sum_k w_k theta_k / sum_k w_k (N, N), loss = mean over r of
    sum_k w_k (theta_k - mean)^2 / sum_k w_k).  Reading, parity unpinned as a
    definition: weighted moments, the loss as the mean variance of the
    pixels' phases."""
    n = n_scan
    s0 = 0.0
    s1 = np.zeros((n, n))
    s2 = np.zeros((n, n))
    for wk, C in pixel_planes(G, k, w, n_scan, step, optics):
        th = np.angle(np.fft.ifft2(C))
        s0 += wk
        s1 += wk * th
        s2 += wk * th * th
    mean = s1 / s0
    var = s2 / s0 - mean * mean
    return mean, float(np.mean(var))


# ----------------------------------------------------------------------------
# compact G: Hermitian half plane as snorm16 pairs with one scale per pixel
# ----------------------------------------------------------------------------

HERM16_ONE = 32767


def herm16_scale(G: np.ndarray, rows: bool = False) -> np.ndarray:
    """float32 scales: the largest |G(q, k)| over each bright-field pixel's
    stored half plane ([P4] compact preview: "per-BF-pixel max |G| over the
    half-plane"), shape (n_bf,); with rows, over each stored row instead
    ([P4] Conclusions: per-q-row block scales, n per pixel), shape (n_bf, N).
    |G|^2 = re^2 + im^2 is formed in float64 from the complex64 components
    (exact squares, one rounding for the sum), the root in float64 and the
    result rounded to float32."""
    G = np.asarray(G)
    re = G.real.astype(np.float64)
    im = G.imag.astype(np.float64)
    m2 = re * re + im * im
    m = m2.max(axis=2) if rows else m2.reshape(G.shape[0], -1).max(axis=1)
    return np.sqrt(m).astype(np.float32)


def _scale_grid(scale: np.ndarray, ndim: int) -> np.ndarray:
    """Scales broadcast against (n_bf, N, N/2+1): per pixel or per row."""
    sd = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return sd.reshape(sd.shape + (1,) * (ndim - sd.ndim))


def herm16_quantize(G: np.ndarray, rows: bool = False):
    """([P4] compact preview: pack2x16snorm(clamp(v / scale))) Each component
    v of G(q, k) becomes the int16 floor(0.5 + 32767 clamp(v / s, -1, 1)),
    the division and the product in float64, each rounded once, s the
    pixel's (or, with rows, the row's) scale; all zero where s = 0.
    Returns (Q int16 (n_bf, N, N/2+1, 2), scale float32 (n_bf,) or
    (n_bf, N))."""
    G = np.asarray(G)
    s = herm16_scale(G, rows)
    sd = _scale_grid(s, G.ndim)
    Q = np.zeros(G.shape + (2,), dtype=np.int16)
    nz = np.broadcast_to(sd > 0, G.shape)
    for c, part in enumerate((G.real, G.imag)):
        v = part.astype(np.float64)
        with np.errstate(invalid="ignore", divide="ignore"):
            x = np.clip(v / sd, -1.0, 1.0)
        q = np.floor(0.5 + HERM16_ONE * x)
        q[~nz] = 0.0
        Q[..., c] = q.astype(np.int16)
    return Q, s


def herm16_dequantize(Q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """G ~ max(q * (1/32767), -1) * s per component, in float64 ([P4]
    compact preview: unpack2x16snorm(word) * scale), s per pixel or per row;
    returns complex128."""
    r = 1.0 / HERM16_ONE
    sd = _scale_grid(scale, Q.ndim - 1)
    re = np.maximum(Q[..., 0].astype(np.float64) * r, -1.0) * sd
    im = np.maximum(Q[..., 1].astype(np.float64) * r, -1.0) * sd
    return re + 1j * im


# ----------------------------------------------------------------------------
# convenience: whole small problems
# ----------------------------------------------------------------------------


def gather_columns(G: np.ndarray, act: np.ndarray, q_list: np.ndarray) -> List[np.ndarray]:
    """G(q, k) over the active pixels for each stored index in q_list."""
    return [np.asarray(G[act, int(iy), int(ix)], dtype=np.complex128) for iy, ix in q_list]


def prepare_all(G: np.ndarray, k: np.ndarray, w: Optional[np.ndarray], n_scan: int, step: float,
                upsampling: int, optics, method: str, smoothness: float, q_list: Optional[np.ndarray] = None):
    """Prepare every unique frequency (or ``q_list``) of a small problem."""
    act = active_pixels(k, optics)
    wa = np.ones(act.shape[0]) if w is None else np.asarray(w, dtype=np.float64)[act]
    if q_list is None:
        q_list = unique_frequencies(n_scan)
    cols = gather_columns(G, act, q_list)
    return prepare(q_list, cols, k[act], wa, n_scan, step, upsampling, optics, method, smoothness)
