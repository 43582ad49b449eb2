"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: numbers the
pages print (tests/golden), textbook closed forms, a brute-force wave-optics
simulation, explicit loops on tiny inputs, and algebraic identities.  Several
tests plant a mistake in the oracle (monkeypatched, CPU only) to show that the
pin would catch it.
"""
import math

import numpy as np
import pytest

from oracle import dsp_oracle as O
from oracle import simulate as S
from synthetic import LAMBDA_300KV, Optics, bf_pixels, workload

LAM = LAMBDA_300KV
ALPHA = 0.030


def tiny_optics(det_step, soft=True):
    return Optics(LAM, ALPHA, det_step, soft=soft, tilt=(2e-3, -1e-3),
                  aberrations=[(1, 0, -50.0, 0.0), (1, 2, 20.0, math.radians(30)),
                               (2, 1, 300.0, 0.4), (3, 0, 1e4, 0.0)])


# ----------------------------------------------------------------------------
# frequency set and aliases
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("n", [4, 8, 32, 128, 512])
def test_unique_set_covers_plane_once(n):
    """U, its conjugates -U and the self-conjugate classes (DC and the Nyquist
    lines) tile the full N x N frequency grid exactly once."""
    U = O.unique_frequencies(n)
    assert len(U) == n * (n - 2) // 2
    cover = np.zeros((n, n), dtype=int)
    for iy, ix in U:
        cover[iy, ix] += 1
        cover[(-iy) % n, (-ix) % n] += 1
    # never solved: DC, the Nyquist row and the Nyquist column
    cover[0, 0] += 1
    cover[n // 2, :] += 1
    cover[:, n // 2] += 1
    cover[n // 2, n // 2] -= 1
    assert np.all(cover == 1)


def test_frequency_count_and_alias_histogram_match_pages(golden):
    g = golden("frequency_counts_512.txt")
    w = workload("c4")
    q, counts, _ = O.alias_table(w.n_scan, w.step, w.upsampling, w.optics)
    assert len(q) == int(g["n_frequencies"][0][0])
    hist = O.alias_histogram(counts)
    want = {int(a): int(b) for a, b in g["alias_count"]}
    assert hist == want
    chunks = sum(math.ceil(v / 128) for v in hist.values())
    assert chunks == int(g["chunks_of_128"][0][0])


def test_alias_histogram_rejects_rival_readings(golden):
    """Plausible mistakes in the alias rule change the printed histogram."""
    g = golden("frequency_counts_512.txt")
    want = {int(a): int(b) for a, b in g["alias_count"]}
    w = workload("c4")
    # hard-aperture radius (no detector-step margin)
    hard = w.optics.replace(soft=False)
    _, c_hard, _ = O.alias_table(w.n_scan, w.step, w.upsampling, hard)
    assert O.alias_histogram(c_hard) != want
    # the rival frequency set "columns 1..N/2-1 and all rows" has the same
    # size but a different histogram
    n = w.n_scan
    dq = O.scan_frequency_step(n, w.step)
    R = O.alias_radius(w.optics)
    rival = [len(O.aliases_of(iy, ix, n, 3, dq, R)) for iy in range(n) for ix in range(1, n // 2)]
    assert len(rival) == 130560
    assert O.alias_histogram(np.asarray(rival)) != want


@pytest.mark.parametrize("u", [1, 2, 3])
def test_alias_rule_bruteforce_tiny(u):
    """Every fine frequency inside the overlap radius is reached exactly once:
    as an alias of a solved frequency or as the conjugate of one (indices
    modulo the fine grid, whose Nyquist lines are their own conjugates);
    fine frequencies of the never-solved classes (DC, coarse Nyquist lines)
    are never reached."""
    n, step = 8, 0.5
    opt = tiny_optics(0.125)
    dq = O.scan_frequency_step(n, step)
    R = O.alias_radius(opt)
    q, counts, Ks = O.alias_table(n, step, u, opt)
    nf = u * n
    seen = {}
    for (iy, ix), K in zip(q, Ks):
        for ky, kx in K:
            assert ((ky - O.signed_index(iy, n)) % n, (kx - ix) % n) == (0, 0)
            assert (ky * ky + kx * kx) * dq * dq < R * R
            for key in {(ky % nf, kx % nf), ((-ky) % nf, (-kx) % nf)}:
                seen[key] = seen.get(key, 0) + 1
    n_inside = 0
    for ky in range(-nf // 2, nf // 2):
        for kx in range(-nf // 2, nf // 2):
            inside = (ky * ky + kx * kx) * dq * dq < R * R
            cy, cx = ky % n, kx % n
            never = (cy == 0 and cx == 0) or cy == n // 2 or cx == n // 2
            hits = seen.get((ky % nf, kx % nf), 0)
            if never:
                assert hits == 0
            elif inside:
                assert hits == 1, (ky, kx)
                n_inside += 1
    assert n_inside > 0


def test_band_count_matches_pages(golden):
    g = golden("band_count_512.txt")
    w = workload("c5")
    m = O.band_mask(w.n_scan, w.step, (float(g["band_lo_invA"][0][0]), float(g["band_hi_invA"][0][0])))
    assert int(m.sum()) == int(g["band_frequencies"][0][0])
    nbf = int(g["bf_pixels"][0][0])
    assert abs(m.sum() * nbf * 8 / 1e9 - float(g["g_band_read_GB"][0][0])) < 0.05
    assert abs(w.n_scan * (w.n_scan // 2 + 1) * nbf * 8 / 1e9 - float(g["g_half_plane_GB"][0][0])) < 0.05


def test_work_counts_match_pages(golden):
    g = golden("magnitudes.txt")
    w = workload("c4")
    _, counts, _ = O.alias_table(w.n_scan, w.step, w.upsampling, w.optics)
    pix, k = bf_pixels(w)
    act = O.active_pixels(k, w.optics)
    assert len(act) == 9298
    pairs = len(act) * int(counts.sum())
    assert abs(pairs / float(g["pixel_alias_pairs"][0][0]) - 1.0) < 0.05
    assert abs(1.0 / w.optics.det_step / float(g["inverse_det_step_A"][0][0]) - 1.0) < 0.05
    assert abs(len(act) * 512 * 257 * 8 / 1e9 - float(g["g_full_frame_GB"][0][0])) < 0.05


# ----------------------------------------------------------------------------
# optics closed forms
# ----------------------------------------------------------------------------


def test_chi_textbook_terms(golden):
    """Defocus, astigmatism, coma and spherical aberration against their
    textbook Cartesian forms; theta = lambda k + tau."""
    rng = np.random.default_rng(3)
    ky, kx = rng.uniform(-1.5, 1.5, size=(2, 50))
    tau = (1.5e-3, -2.5e-3)
    ty, tx = LAM * ky + tau[0], LAM * kx + tau[1]
    t2 = tx * tx + ty * ty
    base = Optics(LAM, ALPHA, 0.03, tilt=tau)
    # defocus C10: pi C10 theta^2 / lambda
    o = base.replace(aberrations=[(1, 0, 120.0, 0.0)])
    assert np.allclose(O.chi(ky, kx, o), math.pi * 120.0 * t2 / LAM, rtol=1e-12, atol=1e-12)
    # two-fold astigmatism C12 at angle p: (pi C12 / lambda)((tx^2 - ty^2) cos 2p + 2 tx ty sin 2p)
    p = 0.7
    o = base.replace(aberrations=[(1, 2, 40.0, p)])
    want = math.pi * 40.0 / LAM * ((tx * tx - ty * ty) * math.cos(2 * p) + 2 * tx * ty * math.sin(2 * p))
    assert np.allclose(O.chi(ky, kx, o), want, rtol=1e-10, atol=1e-12)
    # coma C21 at angle p: (2 pi / 3 lambda) C21 t^2 (tx cos p + ty sin p)
    o = base.replace(aberrations=[(2, 1, 500.0, p)])
    want = 2 * math.pi / (3 * LAM) * 500.0 * t2 * (tx * math.cos(p) + ty * math.sin(p))
    assert np.allclose(O.chi(ky, kx, o), want, rtol=1e-10, atol=1e-12)
    # spherical C30: pi C30 theta^4 / (2 lambda)
    o = base.replace(aberrations=[(3, 0, 1e4, 0.0)])
    assert np.allclose(O.chi(ky, kx, o), math.pi * 1e4 * t2 * t2 / (2 * LAM), rtol=1e-12, atol=1e-12)
    # scale: defocus of 100 A reaches ~14 rad at the 30 mrad edge ("about 13 rad")
    o = Optics(LAM, ALPHA, 0.03, aberrations=[(1, 0, 100.0, 0.0)])
    edge = float(O.chi(ALPHA / LAM, 0.0, o))
    g = golden("magnitudes.txt")
    assert 0.5 < edge / float(g["chi_edge_rad"][0][0]) < 2.0


def test_chi_all_terms_rotate_with_their_angle():
    """chi of term (n, m) at angle phi equals the m-fold rotation of the
    same term at angle 0 (pins the cos(m (p - phi)) angle convention)."""
    rng = np.random.default_rng(4)
    ky, kx = rng.uniform(-1.2, 1.2, size=(2, 20))
    for n, m in [(1, 2), (2, 1), (2, 3), (3, 2), (3, 4), (4, 1), (4, 3), (4, 5), (5, 2), (5, 4), (5, 6)]:
        phi = 0.3
        o1 = Optics(LAM, ALPHA, 0.03, aberrations=[(n, m, 1000.0, phi)])
        o0 = Optics(LAM, ALPHA, 0.03, aberrations=[(n, m, 1000.0, 0.0)])
        c, s = math.cos(-phi), math.sin(-phi)
        # rotate k by -phi: term at angle phi equals term at 0 evaluated there
        kyr, kxr = s * kx + c * ky, c * kx - s * ky
        assert np.allclose(O.chi(ky, kx, o1), O.chi(kyr, kxr, o0), rtol=1e-9, atol=1e-9)


def test_soft_aperture_edge():
    o = Optics(LAM, ALPHA, 0.05, soft=True)
    kc = ALPHA / LAM
    assert O.aperture(kc, o) == pytest.approx(0.5)
    assert O.aperture(kc - 0.025, o) == pytest.approx(1.0)
    assert O.aperture(kc + 0.025, o) == pytest.approx(0.0, abs=1e-12)
    assert O.aperture(kc + 0.0125, o) == pytest.approx(0.25)
    # overlap radius = sum of the two support radii
    assert O.alias_radius(o) == pytest.approx(2 * (kc + 0.025))


# ----------------------------------------------------------------------------
# physics of the transfer: brute-force wave optics
# ----------------------------------------------------------------------------


def _wave_optics_residual(sigma, opt, n=16, step=0.5, u=3, m=96, seed=5):
    rng = np.random.default_rng(seed)
    nf = u * n
    fA = S.band_limited_field(nf, rng)
    fP = S.band_limited_field(nf, rng)
    c = sigma * (fA + 1j * fP)
    k, G = S.wave_optics_G(n, step, m, opt, c, u)
    act = O.active_pixels(k, opt)
    dq = O.scan_frequency_step(n, step)
    q, counts, Ks = O.alias_table(n, step, u, opt)
    FA = S.fine_spectrum(c.real, u)
    FP = S.fine_spectrum(c.imag, u)
    num = den = 0.0
    for (iy, ix), K in zip(q, Ks):
        T = O.transfer(k[act], K * dq, opt, "complex")
        x = np.concatenate([FA[K[:, 0] % nf, K[:, 1] % nf], FP[K[:, 0] % nf, K[:, 1] % nf]])
        model = T @ x
        num += np.sum(np.abs(G[act, iy, ix] - model) ** 2)
        den += np.sum(np.abs(model) ** 2)
    return math.sqrt(num / den), counts


@pytest.mark.parametrize("soft", [True, False])
def test_transfer_matches_wave_optics(soft):
    """The first-order transfer (all alias, lobe, sign and tilt conventions,
    and the aperture, soft or hard) reproduces a brute-force wave-optics
    simulation to O(sigma).  The simulation's probe has its own aperture and
    aberration phase, written from the physics apart from the oracle's."""
    n, step = 16, 0.5
    opt = tiny_optics(O.scan_frequency_step(n, step), soft=soft)
    r1, counts = _wave_optics_residual(1e-3, opt)
    r2, _ = _wave_optics_residual(5e-4, opt)
    assert r1 < 1e-2
    assert 0.4 < r2 / r1 < 0.6           # second-order remainder halves with sigma
    assert len(set(counts.tolist())) > 1  # the tiny case exercises several alias counts


def test_simulator_probe_is_its_own():
    """The simulator imports nothing from the oracle, and its aperture and
    aberration phase agree with the oracle's (two independent codings of the
    same definitions) at scattered points, edge ring and rim included."""
    import inspect

    src = inspect.getsource(S)
    assert "dsp_oracle" not in src and "from ." not in src
    rng = np.random.default_rng(3)
    kc = ALPHA / LAM
    r = np.concatenate([rng.uniform(0, 1.2 * kc, 400), kc + np.array([-0.06, -0.03, 0.0, 0.01, 0.03, 0.06])])
    t = rng.uniform(0, 2 * np.pi, r.size)
    ky, kx = r * np.sin(t), r * np.cos(t)
    for soft in (True, False):
        o = tiny_optics(0.12, soft=soft)
        assert np.array_equal(S.objective_aperture(ky, kx, o) > 0, O.aperture(r, o) > 0)
        assert np.allclose(S.objective_aperture(ky, kx, o), O.aperture(np.hypot(ky, kx), o), rtol=0, atol=1e-12)
        assert np.allclose(S.aberration_phase(ky, kx, o), O.chi(ky, kx, o), rtol=1e-12, atol=1e-9)


def test_hard_aperture_radius_is_pinned(monkeypatch):
    """A hard stop of radius alpha/lambda + dk/2 (the soft support's radius)
    in place of alpha/lambda fails the wave-optics pin and the tiny
    configuration's bright-field count (planted on the CPU only)."""
    n, step = 16, 0.5
    opt = tiny_optics(O.scan_frequency_step(n, step), soft=False)
    true_aperture = O.aperture

    def wide(kabs, optics):
        if optics.soft:
            return true_aperture(kabs, optics)
        return (np.asarray(kabs) <= optics.semiangle / optics.wavelength + 0.5 * optics.det_step).astype(float)

    monkeypatch.setattr(O, "aperture", wide)
    r_bad, _ = _wave_optics_residual(1e-3, opt)
    assert r_bad > 0.05
    assert _c1_bright_field_count() != 113


def _c1_bright_field_count():
    """Active pixels of the tiny SSB configuration's whole 24 x 24 detector
    (hard 30 mrad stop, detector pitch alpha/lambda / 6.04)."""
    w = workload("c1")
    nd = w.n_det
    iy, ix = np.mgrid[0:nd, 0:nd]
    d = np.stack([(iy.ravel() - nd // 2), (ix.ravel() - nd // 2)], axis=1).astype(float) * w.optics.det_step
    return len(O.active_pixels(d, w.optics))


def test_c1_bright_field_count(golden):
    """The tiny SSB configuration's hard stop keeps about 113 of the 24 x 24
    detector pixels (tests/golden/bright_field_counts.txt); brute force over
    the lattice: the integer offsets with dy^2 + dx^2 <= 6.04^2 are 113."""
    want = int(golden("bright_field_counts.txt")["c1_hard_30mrad_24px"][0][0])
    brute = sum(1 for a in range(-12, 12) for b in range(-12, 12) if a * a + b * b <= 6.04 ** 2)
    assert brute == want
    assert _c1_bright_field_count() == want


def test_wave_optics_pin_catches_planted_mistakes(monkeypatch):
    """A plausible convention error in the oracle makes the wave-optics pin
    fail (planted on the CPU only)."""
    n, step = 16, 0.5
    opt = tiny_optics(O.scan_frequency_step(n, step))
    true_lobes = O.lobes

    def swapped(ky, kx, Qy, Qx, optics):
        L, R = true_lobes(ky, kx, Qy, Qx, optics)
        return R, L

    monkeypatch.setattr(O, "lobes", swapped)
    r_bad, _ = _wave_optics_residual(1e-3, opt)
    monkeypatch.setattr(O, "lobes", true_lobes)
    assert r_bad > 0.3

    def no_tilt_shift(ky, kx, Qy, Qx, optics):
        return true_lobes(ky, kx, Qy, Qx, optics.replace(tilt=(0.0, 0.0)))

    monkeypatch.setattr(O, "lobes", no_tilt_shift)
    r_bad, _ = _wave_optics_residual(1e-3, opt)
    assert r_bad > 0.05


# ----------------------------------------------------------------------------
# depth (thick sample): the lobe's sinc and phase factor
# ----------------------------------------------------------------------------


def test_depth_factor_is_the_mean_over_the_slab():
    """depth_factor against brute-force quadrature of exp(i pi z delta / lambda)
    over z in [0, t]; exactly 1 at depth 0."""
    opt = tiny_optics(0.1).replace(depth=80.0)
    delta = np.array([-3e-3, -1e-4, 0.0, 2e-5, 7e-4, 2.5e-3])
    z = (np.arange(20000) + 0.5) / 20000 * opt.depth
    brute = np.exp(1j * math.pi * z[None, :] * delta[:, None] / opt.wavelength).mean(axis=1)
    assert np.allclose(O.depth_factor(delta, opt), brute, rtol=0, atol=1e-8)
    assert np.all(O.depth_factor(delta, opt.replace(depth=0.0)) == 1.0)
    ky, kx = np.array([0.3, -0.5]), np.array([0.1, 0.7])
    L0, R0 = O.lobes(ky, kx, 0.4, -0.2, opt.replace(depth=0.0))
    L1, R1 = O.lobes(ky, kx, 0.4, -0.2, opt.replace(depth=1e-12))
    assert np.allclose(L0, L1, rtol=1e-12, atol=0) and np.allclose(R0, R1, rtol=1e-12, atol=0)


def _depth_residual(sigma, opt, n=16, step=0.5, u=2, m=64, seed=5, n_slices=64):
    rng = np.random.default_rng(seed)
    nf = u * n
    c = sigma * (S.band_limited_field(nf, rng) + 1j * S.band_limited_field(nf, rng))
    k, G = S.wave_optics_G(n, step, m, opt, c, u, n_slices=n_slices)
    act = O.active_pixels(k, opt)
    dq = O.scan_frequency_step(n, step)
    q, _, Ks = O.alias_table(n, step, u, opt)
    FA, FP = S.fine_spectrum(c.real, u), S.fine_spectrum(c.imag, u)
    num = den = 0.0
    for (iy, ix), K in zip(q, Ks):
        T = O.transfer(k[act], K * dq, opt, "complex")
        x = np.concatenate([FA[K[:, 0] % nf, K[:, 1] % nf], FP[K[:, 0] % nf, K[:, 1] % nf]])
        model = T @ x
        num += np.sum(np.abs(G[act, iy, ix] - model) ** 2)
        den += np.sum(np.abs(model) ** 2)
    return math.sqrt(num / den)


def test_depth_transfer_matches_multislice(monkeypatch):
    """The depth terms (sinc and phase factor per lobe, tilt included) against
    a 64-slice multislice simulation of a 60 A weak object; planted mistakes
    (no depth term, conjugated phase factor, sinc without its phase, the
    tilt left out of the depth term) fail by O(1)."""
    n, step = 16, 0.5
    opt = tiny_optics(O.scan_frequency_step(n, step)).replace(depth=60.0)
    r1 = _depth_residual(1e-3, opt)
    r2 = _depth_residual(5e-4, opt)
    assert r1 < 1e-2
    assert 0.4 < r2 / r1 < 0.6
    true_factor = O.depth_factor
    true_lobes = O.lobes
    for name, bad in [
        ("no depth", lambda d, o: np.ones(np.shape(d), dtype=np.complex128)),
        ("conjugate phase", lambda d, o: np.conj(true_factor(d, o))),
        ("sinc only", lambda d, o: np.sinc(0.5 * o.depth * np.asarray(d) / o.wavelength) + 0j),
    ]:
        monkeypatch.setattr(O, "depth_factor", bad)
        r_bad = _depth_residual(1e-3, opt)
        monkeypatch.setattr(O, "depth_factor", true_factor)
        assert r_bad > 0.3, name

    def untilted(ky, kx, Qy, Qx, o):
        L, R = true_lobes(ky, kx, Qy, Qx, o.replace(depth=0.0))
        lam = o.wavelength
        t0 = (lam * ky) ** 2 + (lam * kx) ** 2
        dl = t0 - ((lam * (ky - Qy)) ** 2 + (lam * (kx - Qx)) ** 2)
        dr = (lam * (ky + Qy)) ** 2 + (lam * (kx + Qx)) ** 2 - t0
        return L * true_factor(dl, o), R * true_factor(dr, o)

    monkeypatch.setattr(O, "lobes", untilted)
    r_bad = _depth_residual(1e-3, opt)
    monkeypatch.setattr(O, "lobes", true_lobes)
    assert r_bad > 0.1


# ----------------------------------------------------------------------------
# previews and the loss path
# ----------------------------------------------------------------------------


def _phase_object_data(n=8, step=0.5, sigma=0.05, seed=11, depth=0.0):
    """First-order data of a pure phase object at u = 1 from the simulator's
    probe-amplitude formula (independent of the oracle's lobes)."""
    opt = tiny_optics(O.scan_frequency_step(n, step)).replace(depth=depth)
    rng = np.random.default_rng(seed)
    phi = sigma * S.band_limited_field(n, rng)
    kc = opt.semiangle / opt.wavelength
    k = rng.uniform(-1.1 * kc, 1.1 * kc, size=(40, 2))
    G = S.first_order_G(k, 1j * phi, n, step, 1, opt)
    return opt, phi, k, G


def test_preview_phase_closed_form_for_a_phase_object():
    """Noise-free first-order data of a phase object phi: the corrected sum is
    P(q) = i N(q) Phi(q) with N = sum_k w |Gamma|^2, so the fast path's phase
    is atan2(ifft2(N Phi), D / N^2), D = sum_k w G(0, k).  A conjugation or a
    dropped factor i in the correction fails it."""
    n, step = 8, 0.5
    opt, phi, k, G = _phase_object_data(n, step)
    w = np.linspace(0.5, 1.5, len(k))
    P = O.preview_spectrum(G, k, w, n, step, 1, opt)
    act = O.active_pixels(k, opt)
    ent = np.argwhere(np.ones((n, n // 2 + 1), dtype=bool))
    cols = [np.zeros(len(act), dtype=np.complex128)] * len(ent)
    _, Nh = O.ssb(ent, cols, k[act], w[act], n, step, [opt])
    Nf = np.zeros((n, n))
    Nf[ent[:, 0], ent[:, 1]] = Nh[0]
    for iy in range(n):
        for ix in range(n // 2 + 1, n):
            Nf[iy, ix] = Nf[(-iy) % n, n - ix]      # N(-q) = N(q)
    D = float(np.sum(w[act] * G[act, 0, 0].real))
    want = np.arctan2(np.real(np.fft.ifft2(Nf * np.fft.fft2(phi))), D / (n * n))
    got = O.preview_phase(P)
    assert np.max(np.abs(got - want)) <= 1e-12
    assert np.std(want) > 1e-3                          # a non-trivial image
    true_corrected = O.corrected_term
    for bad in ("conj", "no_i"):
        def planted(ka, wa, Ga, Ky, Kx, n_scan, stp, optics, bad=bad):
            c = true_corrected(ka, wa, Ga, Ky, Kx, n_scan, stp, optics)
            if bad == "conj":   # Gamma instead of conj(Gamma)
                dq = O.scan_frequency_step(n_scan, stp)
                L, R = O.lobes(ka[:, 0], ka[:, 1], Ky * dq, Kx * dq, optics)
                return 1j * wa * (1j * (L - R)) * O.g_full(Ga, Ky, Kx, n_scan)
            return c / 1j
        O.corrected_term = planted
        try:
            bad_phase = O.preview_phase(O.preview_spectrum(G, k, w, n, step, 1, opt))
        finally:
            O.corrected_term = true_corrected
        assert np.max(np.abs(bad_phase - want)) > 0.1 * np.std(want)


def test_preview_at_u1_is_the_ssb_sum():
    """At u = 1 the fast path's spectrum is i S(q) with S the SSB sum at every
    stored q != 0, and sum_k w G(0, k) at DC."""
    w_ = workload("c1")
    n, step = w_.n_scan, w_.step
    opt, _, k, G = _phase_object_data(n=n, step=step, seed=3)
    rng = np.random.default_rng(4)
    G = G + 0.1 * np.fft.rfft2(rng.standard_normal((G.shape[0], n, n)))
    w = rng.uniform(0.5, 1.5, len(k))
    P = O.preview_spectrum(G, k, w, n, step, 1, opt)
    act = O.active_pixels(k, opt)
    ent = np.argwhere(np.ones((n, n // 2 + 1), dtype=bool))
    Sv, _ = O.ssb(ent, [G[act, iy, ix] for iy, ix in ent], k[act], w[act], n, step, [opt])
    Sp = np.zeros((n, n // 2 + 1), dtype=np.complex128)
    Sp[ent[:, 0], ent[:, 1]] = Sv[0]
    Sp[0, 0] = 0.0
    assert not np.any(P[n // 2]) and not np.any(P[:, n // 2])     # the Nyquist lines carry no value
    Sp[n // 2] = 0.0
    Sp[:, n // 2] = 0.0
    assert np.allclose(P[1:], 1j * Sp[1:], rtol=1e-12, atol=1e-12 * np.abs(Sp).max())
    assert np.allclose(P[0, 1:], 1j * Sp[0, 1:], rtol=1e-12, atol=1e-12 * np.abs(Sp).max())
    assert P[0, 0] == pytest.approx(np.sum(w[act] * G[act, 0, 0]), rel=1e-14)


def test_preview_fine_grid_is_the_prepare_rhs():
    """On the u-times finer grid, the corrected sum at an alias K of q equals
    i r_K with r = T_phi^H W g the phase prepare's right side: the fine
    frequency, the G index K mod N and the mirror agree with the alias
    table."""
    n, step, u = 8, 0.5, 3
    opt = tiny_optics(O.scan_frequency_step(n, step))
    rng = np.random.default_rng(6)
    kc = opt.semiangle / opt.wavelength
    k = rng.uniform(-1.1 * kc, 1.1 * kc, size=(30, 2))
    G = np.fft.rfft2(rng.standard_normal((30, n, n)))      # real traces: Hermitian-consistent
    w = rng.uniform(0.5, 1.5, 30)
    P = O.preview_spectrum(G, k, w, n, step, u, opt)
    Fp = O.full_plane(P)
    act = O.active_pixels(k, opt)
    dq = O.scan_frequency_step(n, step)
    q, counts, Ks = O.alias_table(n, step, u, opt)
    m = u * n
    checked = 0
    for (iy, ix), K in zip(q, Ks):
        if len(K) == 0:
            continue
        T = O.transfer(k[act], K * dq, opt, "phase")
        _, r, _ = O.normal_equations(T, G[act, iy, ix], w[act])
        for j, (Ky, Kx) in enumerate(K):
            if Ky == -(m // 2) or abs(Kx) == m // 2:
                continue            # the fine grid's Nyquist lines carry no value
            got = Fp[Ky % m, Kx % m]
            assert abs(got - 1j * r[j]) <= 1e-11 * max(1.0, abs(r[j])), (iy, ix, Ky, Kx)
            checked += 1
    assert checked > 100


def test_preview_is_antihermitian_off_dc():
    """Direct evaluation at K and -K: P(-K) = -conj P(K) for K != 0 ([P3] Open:
    the corrected spectrum of a real image)."""
    n, step, u = 8, 0.5, 2
    opt = tiny_optics(O.scan_frequency_step(n, step)).replace(depth=60.0)
    rng = np.random.default_rng(7)
    kc = opt.semiangle / opt.wavelength
    k = rng.uniform(-1.1 * kc, 1.1 * kc, size=(25, 2))
    G = np.fft.rfft2(rng.standard_normal((25, n, n)))
    w = rng.uniform(0.5, 1.5, 25)
    act = O.active_pixels(k, opt)
    for Ky, Kx in [(1, 2), (-3, 5), (7, -6), (0, 3), (-8, 1), (5, 8)]:
        a = np.sum(O.corrected_term(k[act], w[act], G[act], Ky, Kx, n, step, opt))
        b = np.sum(O.corrected_term(k[act], w[act], G[act], -Ky, -Kx, n, step, opt))
        assert abs(b + np.conj(a)) <= 1e-12 * max(1.0, abs(a))


def test_fast_path_identity_and_single_pixel_loss():
    """[P4]'s identity: the mean of the pixels' objects is the inverse FFT of
    the summed corrected planes, so angle(sum_k o_k) is the fast path's
    phase; with one pixel, mean(angle) = angle(mean) and the loss is 0.  A
    pixel's object by explicit DFT double sums (e^{+2 pi i q.r} / N^2) equals
    the inverse FFT."""
    n, step = 8, 0.5
    opt, _, k, G = _phase_object_data(n, step, seed=12)
    w = np.linspace(0.7, 1.3, len(k))
    objs = [np.fft.ifft2(C) for _, C in O.pixel_planes(G, k, w, n, step, opt)]
    fast = O.preview_phase(O.preview_spectrum(G, k, w, n, step, 1, opt))
    assert np.max(np.abs(np.angle(np.sum(objs, axis=0)) - fast)) <= 1e-12
    # explicit DFT of one pixel's plane; the plane is anti-Hermitian off DC,
    # so its object is C(0) / N^2 + i (a real image)
    _, C0 = next(iter(O.pixel_planes(G, k, w, n, step, opt)))
    mirror = -np.conj(C0[(-np.arange(n)) % n][:, (-np.arange(n)) % n])
    mirror[0, 0] = C0[0, 0]
    assert np.allclose(C0, mirror, rtol=0, atol=1e-12 * np.abs(C0).max())
    assert np.allclose(objs[0].real, C0[0, 0].real / n ** 2, rtol=0, atol=1e-12 * np.abs(objs[0]).max())
    r = np.arange(n)
    E = np.exp(2j * math.pi * np.outer(r, r) / n)
    brute = (E @ C0 @ E.T) / (n * n)
    assert np.allclose(brute, objs[0], rtol=0, atol=1e-12 * np.abs(objs[0]).max())
    # one pixel
    act = O.active_pixels(k, opt)
    k1 = k[act[:1]]
    G1 = G[act[:1]]
    mean, loss = O.loss_path(G1, k1, None, n, step, opt)
    assert loss == pytest.approx(0.0, abs=1e-15)
    assert np.max(np.abs(mean - O.preview_phase(O.preview_spectrum(G1, k1, None, n, step, 1, opt)))) <= 1e-12


def test_loss_is_a_weighted_variance():
    """The loss against explicit per-pixel phases: the weighted variance about
    the weighted mean, averaged over the scan; zero-weight pixels drop out."""
    n, step = 8, 0.5
    opt, _, k, G = _phase_object_data(n, step, seed=13)
    rng = np.random.default_rng(14)
    G = G + 0.5 * np.fft.rfft2(rng.standard_normal((G.shape[0], n, n)))
    w = rng.uniform(0.5, 1.5, len(k))
    w[::4] = 0.0
    th, ws = [], []
    for wk, C in O.pixel_planes(G, k, w, n, step, opt):
        th.append(np.angle(np.fft.ifft2(C)))
        ws.append(wk)
    th = np.array(th)
    ws = np.array(ws)
    keep = ws > 0
    mean_b = np.average(th[keep], axis=0, weights=ws[keep])
    var_b = np.average((th[keep] - mean_b) ** 2, axis=0, weights=ws[keep])
    mean, loss = O.loss_path(G, k, w, n, step, opt)
    assert np.allclose(mean, mean_b, rtol=0, atol=1e-13)
    assert loss == pytest.approx(float(var_b.mean()), rel=1e-9)
    assert loss > 1e-4


# ----------------------------------------------------------------------------
# compact G (herm16)
# ----------------------------------------------------------------------------


def test_herm16_error_bound_and_exact_values():
    """Each dequantized component is within half a quantization step of the
    original (round to nearest; truncation would reach a full step), values
    on the grid round-trip exactly, the scale is the plane's largest |G|, and
    an all-zero plane stays zero."""
    rng = np.random.default_rng(3)
    G = (rng.standard_normal((5, 8, 5)) + 1j * rng.standard_normal((5, 8, 5))).astype(np.complex64)
    G[1] *= 1e-6                       # pixels of very different magnitude
    G[3] = 0
    Q, s = O.herm16_quantize(G)
    assert Q.dtype == np.int16 and s.dtype == np.float32
    mag = np.abs(G.astype(np.complex128)).reshape(5, -1).max(axis=1)
    assert np.allclose(s, mag, rtol=1e-7, atol=0)
    assert not np.any(Q[3]) and s[3] == 0
    D = O.herm16_dequantize(Q, s)
    step = s.astype(np.float64)[:, None, None] / 32767.0
    assert np.all(np.abs(D.real - G.real) <= 0.5 * step * (1 + 1e-9) + 1e-300)
    assert np.all(np.abs(D.imag - G.imag) <= 0.5 * step * (1 + 1e-9) + 1e-300)
    # the largest component of each pixel maps to +-32767 (the scale is |G|,
    # so only a purely real or imaginary maximum reaches the end points)
    assert np.abs(Q).max() <= 32767
    grid = np.zeros((1, 2, 2), dtype=np.complex64)
    grid[0, 0, 0] = 1.0
    grid[0, 1, 1] = -0.5 + 0.25j
    Qg, sg = O.herm16_quantize(grid)
    assert sg[0] == 1.0 and Qg[0, 0, 0, 0] == 32767 and Qg[0, 1, 1, 0] == -16383 and Qg[0, 1, 1, 1] == 8192


def test_herm16_row_scales():
    """Per-row scales: each is its row's largest |G|, the error stays within
    half a step of that row's scale (never more than the per-pixel bound),
    an all-zero row packs to zeros, and a row of one known value round-trips
    at its codes."""
    rng = np.random.default_rng(4)
    n = 8
    G = np.fft.rfft2(rng.standard_normal((3, n, n))).astype(np.complex64)
    G[:, :, 0] *= 50.0                     # a strong column, as DC-dominated planes have
    G[2, 5] = 0
    Q, s = O.herm16_quantize(G, rows=True)
    assert s.shape == (3, n) and s.dtype == np.float32
    mag = np.abs(G.astype(np.complex128)).max(axis=2)
    assert np.allclose(s, mag, rtol=1e-7, atol=0)
    assert s[2, 5] == 0 and not np.any(Q[2, 5])
    D = O.herm16_dequantize(Q, s)
    step = s.astype(np.float64)[:, :, None] / 32767.0
    assert np.all(np.abs(D.real - G.real) <= 0.5 * step * (1 + 1e-9) + 1e-300)
    assert np.all(np.abs(D.imag - G.imag) <= 0.5 * step * (1 + 1e-9) + 1e-300)
    _, s_pix = O.herm16_quantize(G)
    assert np.all(s <= s_pix[:, None])
    err_rows = np.abs(D - G).max()
    err_pix = np.abs(O.herm16_dequantize(*O.herm16_quantize(G)) - G).max()
    assert err_rows < err_pix
    one = np.zeros((1, 2, 2), dtype=np.complex64)
    one[0, 1, :] = [0.5 - 0.25j, -1.0 + 0.0j]
    Qo, so = O.herm16_quantize(one, rows=True)
    assert so[0, 1] == 1.0 and so[0, 0] == 0.0
    assert list(Qo[0, 1, 0]) == [16384, -8192] and list(Qo[0, 1, 1]) == [-32767, 0]


def test_first_order_model_equals_transfer_sum():
    """The physics-form first-order data (written from A(k)) equals
    sum_Q T x over the oracle's aliases."""
    n, step, u = 8, 0.5, 3
    opt = tiny_optics(0.1)
    rng = np.random.default_rng(9)
    nf = u * n
    c = 0.01 * (S.band_limited_field(nf, rng) + 1j * S.band_limited_field(nf, rng))
    w = workload("c1")
    _, k = bf_pixels(w)
    k = k * 0.1 / w.optics.det_step  # spread over the aperture at this dk
    act = O.active_pixels(k, opt)
    G = S.first_order_G(k[act], c, n, step, u, opt, include_dc=False)
    dq = O.scan_frequency_step(n, step)
    q, _, Ks = O.alias_table(n, step, u, opt)
    FA, FP = S.fine_spectrum(c.real, u), S.fine_spectrum(c.imag, u)
    for (iy, ix), K in zip(q, Ks):
        T = O.transfer(k[act], K * dq, opt, "complex")
        x = np.concatenate([FA[K[:, 0] % nf, K[:, 1] % nf], FP[K[:, 0] % nf, K[:, 1] % nf]])
        assert np.allclose(G[:, iy, ix], T @ x, rtol=1e-12, atol=1e-12 * np.abs(G).max())


# ----------------------------------------------------------------------------
# normal equations and solves
# ----------------------------------------------------------------------------


def _small_problem(method, u=2, n=8, seed=0, weights=True):
    step = 0.5
    opt = tiny_optics(0.12)
    rng = np.random.default_rng(seed)
    ang = rng.uniform(0, 2 * np.pi, 60)
    rad = np.sqrt(rng.uniform(0, 1, 60)) * (ALPHA / LAM + 0.05)
    k = np.stack([rad * np.sin(ang), rad * np.cos(ang)], axis=1)
    act = O.active_pixels(k, opt)
    k = k[act]
    w = rng.uniform(0.5, 1.5, len(k)) if weights else np.ones(len(k))
    q = O.unique_frequencies(n)
    cols = [rng.standard_normal(len(k)) + 1j * rng.standard_normal(len(k)) for _ in q]
    prep = O.prepare(q, cols, k, w, n, step, u, opt, method, smoothness=ALPHA / LAM)
    return prep, k, w, cols, opt, n, step, u


def test_gram_bruteforce_loops():
    """Gram, right side and power by explicit Python loops over pixels and
    unknowns, transfer entries from the lobe definitions one pixel at a time."""
    prep, k, w, cols, opt, n, step, u = _small_problem("complex")
    dq = O.scan_frequency_step(n, step)
    kc = ALPHA / LAM

    def amp(y, x):
        return min(1.0, max(0.0, 0.5 + (kc - math.hypot(y, x)) / opt.det_step))

    def phase(y, x):
        ty, tx = LAM * y + opt.tilt[0], LAM * x + opt.tilt[1]
        t, p = math.hypot(ty, tx), math.atan2(ty, tx)
        return 2 * math.pi / LAM * sum(c * t ** (nn + 1) / (nn + 1) * math.cos(mm * (p - ph))
                                        for nn, mm, c, ph in opt.aberrations)

    for i in [0, 5, len(prep.q) - 1]:
        K = prep.K[i]
        A = K.shape[0]
        T = np.zeros((len(k), 2 * A), dtype=complex)
        for j, (y, x) in enumerate(k):
            for m in range(A):
                Qy, Qx = K[m, 0] * dq, K[m, 1] * dq
                L = amp(y, x) * amp(y - Qy, x - Qx) * np.exp(1j * (phase(y, x) - phase(y - Qy, x - Qx)))
                R = amp(y, x) * amp(y + Qy, x + Qx) * np.exp(-1j * (phase(y, x) - phase(y + Qy, x + Qx)))
                T[j, m] = L + R
                T[j, A + m] = 1j * (L - R)
        d = 2 * A
        M = np.zeros((d, d), dtype=complex)
        r = np.zeros(d, dtype=complex)
        P = 0.0
        for j in range(len(k)):
            for a in range(d):
                r[a] += w[j] * np.conj(T[j, a]) * cols[i][j]
                for b in range(d):
                    M[a, b] += w[j] * np.conj(T[j, a]) * T[j, b]
            P += w[j] * abs(cols[i][j]) ** 2
        assert np.allclose(prep.M[i], M, rtol=1e-12, atol=1e-12 * abs(M).max())
        assert np.allclose(prep.r[i], r, rtol=1e-12, atol=1e-12 * abs(r).max())
        assert prep.P[i] == pytest.approx(P, rel=1e-13)


def test_gram_hermitian_psd():
    prep, *_ = _small_problem("complex", u=3)
    for M, r, P in zip(prep.M, prep.r, prep.P):
        assert np.abs(M - M.conj().T).max() <= 1e-15 * max(1.0, np.abs(M).max())
        aug = np.block([[M, r[:, None]], [r.conj()[None, :], np.array([[P]])]])
        ev = np.linalg.eigvalsh(aug)
        assert ev.min() >= -1e-12 * ev.max()


def test_eigenbasis_equals_direct_solve():
    prep, *_ = _small_problem("phase", u=3)
    for s in [1e-3, 1e-1, 3.0]:
        xe = O.solve(prep, s, use_eigenbasis=True)
        xd = O.solve(prep, s, use_eigenbasis=False)
        for a, b in zip(xe, xd):
            assert np.linalg.norm(a - b) <= 1e-11 * max(np.linalg.norm(b), 1e-300)
    for lam in prep.lam:
        assert np.all(np.diff(lam) >= 0)


def test_complex_system_contains_phase_system():
    pc, *_ = _small_problem("complex", u=3, seed=2)
    pp, *_ = _small_problem("phase", u=3, seed=2)
    for Mc, rc, Mp, rp, A in zip(pc.M, pc.r, pp.M, pp.r, pc.A):
        assert np.allclose(Mc[A:, A:], Mp, rtol=0, atol=1e-15 * np.abs(Mc).max())
        assert np.allclose(rc[A:], rp, rtol=0, atol=1e-15 * np.abs(rc).max())


@pytest.mark.parametrize("method", ["phase", "complex"])
def test_solution_minimizes_objective(method):
    """x(lambda) minimizes sum_k w |g - T x|^2 + lambda scale sum p |x|^2,
    evaluated by brute force; and the residual identity holds."""
    prep, k, w, cols, opt, n, step, u = _small_problem(method, u=3, seed=4)
    dq = O.scan_frequency_step(n, step)
    strength = 0.05 if method == "phase" else (0.05, 0.02)
    xs = O.solve(prep, strength)
    rng = np.random.default_rng(1)
    for i in [1, 7, 20]:
        T = O.transfer(k, prep.K[i] * dq, opt, method)
        g = cols[i]
        A = prep.A[i]
        if method == "phase":
            reg = strength * prep.scale * prep.p[i]
        else:
            reg = prep.scale * np.concatenate([strength[0] * prep.p[i][:A], strength[1] * prep.p[i][A:]])

        def J(x):
            return np.sum(w * np.abs(g - T @ x) ** 2) + np.sum(reg * np.abs(x) ** 2)

        x = xs[i]
        j0 = J(x)
        for _ in range(5):
            d = rng.standard_normal(x.shape) + 1j * rng.standard_normal(x.shape)
            d *= 1e-3 * np.linalg.norm(x) / np.linalg.norm(d)
            assert J(x + d) > j0 and J(x - d) > j0
        rho = np.sum(w * np.abs(g - T @ x) ** 2)
        assert O.residual(prep.M[i], prep.r[i], prep.P[i], x) == pytest.approx(rho, rel=1e-10)


def test_planted_transpose_breaks_minimality(monkeypatch):
    """Using M^T instead of M in the solve is caught by the objective pin."""
    prep, k, w, cols, opt, n, step, u = _small_problem("complex", u=3, seed=4)
    prep.M = [M.T for M in prep.M]
    xs = O.solve(prep, (0.05, 0.05))
    dq = O.scan_frequency_step(n, step)
    i = 7
    T = O.transfer(k, prep.K[i] * dq, opt, "complex")
    A = prep.A[i]
    reg = prep.scale * 0.05 * np.concatenate([prep.p[i][:A], prep.p[i][A:]])
    x_true = np.linalg.solve(T.conj().T @ (w[:, None] * T) + np.diag(reg), T.conj().T @ (w * cols[i]))
    assert np.linalg.norm(xs[i] - x_true) > 1e-6 * np.linalg.norm(x_true)


def _prior_deviation(method):
    """The prior as the solve applies it, read back from the solution: with
    x = (M + mu D)^-1 r (mu = strength x scale, per component for complex),
    D x = (r - M x) / mu, so p_j = (r - M x)_j / (mu_j x_j) at every unknown.
    Returns the largest relative deviation of p from the pages' printed prior
    (1 + q^2/s^2)^2 ("Where the 9 s of regularized preparation goes", Raw
    numbers, the prior stage; tests/golden/prior.txt) taken at each alias's
    own fine frequency |Q| = |K| dq, over a three-times upsampled tiny scan
    whose aliases of one scan frequency lie at different |Q|."""
    n, step, u = 12, 0.45, 3
    opt = tiny_optics(0.1)
    rng = np.random.default_rng(31)
    w = workload("c2")
    _, k = bf_pixels(w)
    k = k[O.active_pixels(k, opt)]
    q = O.unique_frequencies(n)
    cols = [rng.standard_normal(len(k)) + 1j * rng.standard_normal(len(k)) for _ in q]
    wts = rng.uniform(0.5, 1.5, len(k))
    s_p = 1.3                         # |Q| / s_p spans about 0 to 3 over the aliases
    prep = O.prepare(q, cols, k, wts, n, step, u, opt, method, smoothness=s_p)
    dq = O.scan_frequency_step(n, step)
    st = 0.2 if method == "phase" else (0.2, 0.35)
    xs = O.solve(prep, st)
    worst, n_diff = 0.0, 0
    for i, x in enumerate(xs):
        A = int(prep.A[i])
        if A == 0:
            continue
        Q = prep.K[i] * dq
        t2 = (Q[:, 0] ** 2 + Q[:, 1] ** 2) / s_p ** 2
        printed = (1.0 + t2) ** 2
        if method == "phase":
            mu = st * prep.scale * np.ones(A)
            want = printed
        else:
            mu = prep.scale * np.concatenate([st[0] * np.ones(A), st[1] * np.ones(A)])
            want = np.concatenate([printed, printed])
        p_back = (prep.r[i] - prep.M[i] @ x) / (mu * x)
        assert np.abs(p_back.imag).max() <= 1e-6 * np.abs(p_back.real).max()
        worst = max(worst, float(np.abs(p_back.real - want).max() / want.max()))
        n_diff += int(np.ptp(printed) > 0.1)
    assert n_diff > 10                # aliases of one frequency see different priors
    return worst


@pytest.mark.parametrize("method", ["phase", "complex"])
def test_prior_through_the_solve(method, golden):
    """The prior the solve applies, recovered from its solutions, is the
    printed (1 + q^2/s^2)^2 at each alias's fine |Q|."""
    assert golden("prior.txt")["exponent"][0][0] == "2"
    assert _prior_deviation(method) <= 1e-6


def test_prior_mistakes_are_caught(monkeypatch):
    """Planted on the CPU: a prior of power 1, or one taken at the coarse scan
    frequency instead of the alias's fine |Q|, fails the solve pin."""
    true_prior = O.prior

    def power_one(Q, s):
        return np.sqrt(true_prior(Q, s))

    monkeypatch.setattr(O, "prior", power_one)
    assert _prior_deviation("phase") > 1e-2
    n, step = 12, 0.45
    period = n * O.scan_frequency_step(n, step)

    def coarse(Q, s):
        Qc = (np.asarray(Q) / period + 0.5) % 1.0 - 0.5
        return true_prior(Qc * period, s)

    monkeypatch.setattr(O, "prior", coarse)
    assert _prior_deviation("complex") > 1e-2


# ----------------------------------------------------------------------------
# closed-form recovery and scatter
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("method", ["phase", "complex"])
def test_noise_free_recovery_and_scatter(method):
    """Noise-free first-order data from a known object: the prepared system
    returns x = (M + mu D)^-1 M x_true and, as mu -> 0, x_true on every
    well-conditioned frequency; the scatter places it at fft2(c)/u^2."""
    n, step, u = 16, 0.5, 2
    opt = tiny_optics(0.125)
    rng = np.random.default_rng(11)
    nf = u * n
    phi = S.band_limited_field(nf, rng, std=0.05)
    amp = S.band_limited_field(nf, rng, std=0.02) if method == "complex" else np.zeros_like(phi)
    c = amp + 1j * phi
    w = workload("c2")
    _, k = bf_pixels(w)
    act = O.active_pixels(k, opt)
    k = k[act]
    G = S.first_order_G(k, c, n, step, u, opt)
    q = O.unique_frequencies(n)
    cols = [G[:, iy, ix] for iy, ix in q]
    wts = np.ones(len(k))
    prep = O.prepare(q, cols, k, wts, n, step, u, opt, method, smoothness=ALPHA / LAM)
    FA, FP = S.fine_spectrum(amp, u), S.fine_spectrum(phi, u)
    tiny = 1e-10 if method == "phase" else (1e-10, 1e-10)
    xs = O.solve(prep, tiny)
    checked = 0
    x_true_all = []
    for i, K in enumerate(prep.K):
        xt = FP[K[:, 0] % nf, K[:, 1] % nf]
        if method == "complex":
            xt = np.concatenate([FA[K[:, 0] % nf, K[:, 1] % nf], xt])
        x_true_all.append(xt)
        M = prep.M[i]
        ev = np.linalg.eigvalsh(M)
        if ev[0] > 1e-6 * ev[-1]:
            assert np.linalg.norm(xs[i] - xt) <= 1e-6 * np.linalg.norm(xt) + 1e-12
            checked += 1
        # moderate strength: closed form of Tikhonov on exact data
        s = 0.1 if method == "phase" else (0.1, 0.1)
        xm = O.solve(prep, s)[i] if i < 3 else None
        if xm is not None:
            mu = 0.1 * prep.scale
            want = np.linalg.solve(M + np.diag(mu * prep.p[i]), M @ xt)
            assert np.allclose(xm, want, rtol=1e-9, atol=1e-12)
    assert checked > 0.8 * len(prep.K)
    ncomp = 2 if method == "complex" else 1
    spec = O.scatter(prep.q, prep.K, x_true_all, n, u, ncomp)
    want = [FA, FP] if method == "complex" else [FP]
    for c_i in range(ncomp):
        sp = spec[c_i]
        ref = want[c_i][:, : nf // 2 + 1]
        nz = sp != 0
        assert np.allclose(sp[nz], ref[nz], rtol=1e-12, atol=1e-15)
        # the fine real-field spectrum is recovered wherever an alias reaches it
        assert nz.sum() > 0.5 * nz.size


# ----------------------------------------------------------------------------
# SSB sum and agreement
# ----------------------------------------------------------------------------


def test_ssb_equals_unregularized_prepare_at_u1():
    """At one alias per frequency with no prior and zero strength, S/N is the
    prepared solution."""
    w = workload("c1")
    pix, k = bf_pixels(w)
    opt = w.optics
    act = O.active_pixels(k, opt)
    rng = np.random.default_rng(2)
    q = O.unique_frequencies(w.n_scan)[::7]
    cols = [rng.standard_normal(len(act)) + 1j * rng.standard_normal(len(act)) for _ in q]
    wts = rng.uniform(0.5, 1.5, len(act))
    prep = O.prepare(q, cols, k[act], wts, w.n_scan, w.step, 1, opt, "phase", smoothness=0.0)
    Sv, Nv = O.ssb(q, cols, k[act], wts, w.n_scan, w.step, [opt])
    n_ok = 0
    for i in range(len(q)):
        if Nv[0, i] > 1e-9 * Nv.max():
            x = O.solve_direct(prep.M[i], prep.r[i], np.zeros(1))
            assert abs(Sv[0, i] / Nv[0, i] - x[0]) <= 1e-12 * abs(x[0]) + 1e-15
            n_ok += 1
    assert n_ok > 0.5 * len(q)


def test_agreement_is_maximal_at_true_optics():
    """Noise-free single-alias data: the agreement peaks at the true defocus
    and stays <= 1."""
    n, step = 16, 0.5
    opt = Optics(LAM, ALPHA, 0.1, soft=True, aberrations=[(1, 0, -60.0, 0.0), (3, 0, 1e4, 0.0)])
    rng = np.random.default_rng(8)
    phi = S.band_limited_field(n, rng, std=0.05, cutoff=0.6)
    w = workload("c1")
    _, k = bf_pixels(w)
    k = k * 0.1 / w.optics.det_step
    act = O.active_pixels(k, opt)
    k = k[act]
    G = S.first_order_G(k, 1j * phi, n, step, 1, opt)
    wts = np.ones(len(k))
    entries = np.argwhere(O.band_mask(n, step, (0.2, 0.9)))
    cols = [G[:, iy, ix] for iy, ix in entries]
    power = np.array([np.sum(wts * np.abs(g) ** 2) for g in cols])
    shifts = [-20.0, -10.0, -5.0, 0.0, 5.0, 10.0, 20.0]
    sets = [opt.replace(aberrations=[(1, 0, -60.0 + d, 0.0), (3, 0, 1e4, 0.0)]) for d in shifts]
    Sv, Nv = O.ssb(entries, cols, k, wts, n, step, sets)
    E = O.agreement(Sv, Nv, power)
    assert np.argmax(E) == shifts.index(0.0)
    assert E[shifts.index(0.0)] == pytest.approx(1.0, abs=1e-9)
    assert np.all(np.diff(E[:4]) > 0) and np.all(np.diff(E[3:]) < 0)


def test_bright_field_sum_linearity():
    """Summing corrected G over pixels then one inverse FFT equals the mean of
    per-pixel inverse FFTs ([P4] object-redraw identity)."""
    rng = np.random.default_rng(0)
    G = rng.standard_normal((5, 8, 8)) + 1j * rng.standard_normal((5, 8, 8))
    corr = np.exp(1j * rng.uniform(0, 6.3, (5, 8, 8)))
    a = np.fft.ifft2((G * corr).sum(axis=0)) / 5
    b = np.mean([np.fft.ifft2(G[i] * corr[i]) for i in range(5)], axis=0)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
