"""GPU tests at the limits: the alias-slot maximum, a bright-field set with no
active pixel, the largest supported scan (N = 8192) against the oracle on
sampled outputs and exact properties, and the loss path's fused transforms
at their smallest and largest scans."""
import math

import numpy as np
import pytest

from oracle import dsp_oracle as O
from synthetic import LAMBDA_300KV, Optics

torch = pytest.importorskip("torch")
dsp = pytest.importorskip("stem_direct_ptychography_amd")
from stem_direct_ptychography_amd import _lib  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
X_TOL = 1e-5


def _say(msg):
    print(f"[gpu-edges] {msg}", flush=True)


def _optics(soft=True, det_step=0.05, depth=0.0):
    return Optics(LAMBDA_300KV, 0.03, det_step, soft=soft, tilt=(1e-3, -2e-3), depth=depth,
                  aberrations=[(1, 0, -60.0, 0.0), (1, 2, 15.0, 0.4), (3, 0, 2e4, 0.0)])


def _pixels(opt, n, seed):
    kc = opt.semiangle / opt.wavelength
    rng = np.random.default_rng(seed)
    r = kc * np.sqrt(rng.uniform(0.0, 0.8, n))
    a = rng.uniform(0.0, 2.0 * math.pi, n)
    return np.stack([r * np.sin(a), r * np.cos(a)], axis=1)


class _Columns:
    """G[:, iy, ix] for a few stored entries, for oracle calls that read one
    entry of a full-size plane."""

    def __init__(self, cols):
        self.cols = cols

    def __getitem__(self, key):
        _, iy, ix = key
        return self.cols[(int(iy), int(ix))]


def _real_stack(n_bf, n, seed):
    """G of real intensity traces (Hermitian-consistent), complex64 on the GPU."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    return torch.fft.rfft2(torch.randn((n_bf, n, n), generator=gen, device=DEV)).contiguous()


def test_alias_slot_limit():
    """A scan step coarse enough that every fine alias of a frequency lies in
    reach: 9 aliases at u = 3 exceed both methods' slot maxima (8 phase,
    6 complex) and the prepare says so; u = 2 (4 aliases) runs."""
    opt = _optics()
    n, step = 8, 1.5
    _, counts, _ = O.alias_table(n, step, 3, opt)
    assert counts.max() == 9
    k = _pixels(opt, 12, 1)
    G = _real_stack(12, n, 2)
    for method in ("phase", "complex"):
        with pytest.raises(dsp.DspError) as e:
            dsp.prepare(G, k, opt, step=step, upsampling=3, method=method)
        assert e.value.status == _lib.DSP_EALIAS, method
        p = dsp.prepare(G, k, opt, step=step, upsampling=2, method=method)
        assert p.info["a_max"] == 4
        del p


def test_no_active_pixel():
    """Pixels all outside the aperture: every pass over G refuses them."""
    opt = _optics(soft=False)
    kc = opt.semiangle / opt.wavelength
    k = np.array([[2.0 * kc, 0.0], [0.0, -1.5 * kc], [1.2 * kc, 1.2 * kc]])
    n, step = 16, 0.5
    G = _real_stack(3, n, 3)
    calls = [lambda: dsp.prepare(G, k, opt, step=step, upsampling=1, method="phase"),
             lambda: dsp.ssb(G, k, [opt], step=step),
             lambda: dsp.preview(G, k, opt, step=step),
             lambda: dsp.loss(G, k, opt, step=step)]
    for call in calls:
        with pytest.raises(dsp.DspError) as e:
            call()
        assert e.value.status == _lib.DSP_EINVAL


def test_largest_scan():
    """N = 8192 (33.5 million solved frequencies at u = 1) with three pixels:
    sampled phase solutions and SSB entries against the oracle, the preview's
    sampled fine entries and DC, and the loss path's mean phase of the three
    pixels against the mean of three one-pixel runs."""
    n, step = 8192, 0.373
    opt = _optics(soft=False, det_step=0.02819)
    k = _pixels(opt, 3, 4)
    _say("G (3, 8192, 4097) complex64 from real traces")
    G = _real_stack(3, n, 5)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    # sampled solved frequencies (stored iy, ix with ix < N/2, iy != N/2, not ix = 0 with row <= 0)
    picks = []
    while len(picks) < 24:
        iy, ix = int(rng.integers(0, n)), int(rng.integers(1, n // 2))
        if iy != n // 2:
            picks.append((iy, ix))
    picks = np.array(sorted(picks))
    _say("phase prepare at N = 8192 (host geometry takes several seconds)")
    prep = dsp.prepare(G, k, opt, step=step, upsampling=1, method="phase", smoothness=0.0)
    x = prep.solve([1e-2]).cpu().numpy()[0, 0, :, 0]
    q, _, _ = prep.alias_table()
    assert len(q) == n * (n - 2) // 2
    key = q[:, 0].astype(np.int64) * n + q[:, 1]          # the solved list is row-major
    pos = np.searchsorted(key, picks[:, 0].astype(np.int64) * n + picks[:, 1])
    assert np.array_equal(q[pos], picks)
    del q, key
    _say("oracle on the sampled frequencies")
    act = O.active_pixels(k, opt)
    Gp = G[:, torch.as_tensor(picks[:, 0], device=DEV), torch.as_tensor(picks[:, 1], device=DEV)]
    Gp = Gp.cpu().numpy().astype(np.complex128)
    cols = [Gp[act, j] for j in range(len(picks))]
    prep_o = O.prepare(picks, cols, k[act], np.ones(len(act)), n, step, 1, opt, "phase", 0.0)
    xs_o = O.solve(prep_o, 1e-2)
    for j, (iy, ix) in enumerate(picks):
        i = pos[j]
        want = xs_o[j][0]
        assert abs(x[i] - want) <= X_TOL * max(abs(want), 1e-12), (iy, ix)
    del prep
    _say("SSB over the 0.2-0.9 1/A band")
    S, Nn, _ = dsp.ssb(G, k, [opt], step=step, band=(0.2, 0.9), agreement=False)
    S = S.cpu().numpy()
    Nn = Nn.cpu().numpy()
    mask_pick = []
    dq = O.scan_frequency_step(n, step)
    while len(mask_pick) < 24:
        iy, ix = int(rng.integers(0, n)), int(rng.integers(0, n // 2 + 1))
        f = math.hypot(float(O.signed_index(iy, n)) * dq, ix * dq)
        if 0.2 <= f <= 0.9:
            mask_pick.append((iy, ix))
    ent = np.array(mask_pick)
    Ge = G[:, torch.as_tensor(ent[:, 0], device=DEV), torch.as_tensor(ent[:, 1], device=DEV)].cpu().numpy()
    S_o, N_o = O.ssb(ent, [Ge[act, j].astype(np.complex128) for j in range(len(ent))], k[act], np.ones(len(act)),
                     n, step, [opt])
    got = S[0, ent[:, 0], ent[:, 1]]
    assert np.max(np.abs(got - S_o[0]) / np.maximum(np.abs(S_o[0]), 1e-3 * np.abs(S_o[0]).max())) <= X_TOL
    assert np.allclose(Nn[0, ent[:, 0], ent[:, 1]], N_o[0], rtol=X_TOL, atol=0)
    del S, Nn
    _say("preview at u = 1")
    P, _ = dsp.preview(G, k, opt, step=step, upsampling=1, phase=False)
    P = P.cpu().numpy()
    for j, (iy, ix) in enumerate(mask_pick[:8]):
        Ky = int(O.signed_index(iy, n))
        cols = _Columns({(iy, ix): Ge[act, j].astype(np.complex128)})
        want = np.sum(O.corrected_term(k[act], np.ones(len(act)), cols, Ky, ix, n, step, opt))
        assert abs(P[iy, ix] - want) <= X_TOL * max(abs(want), 1e-12), (iy, ix)
    dc = np.sum(G[torch.as_tensor(act, device=DEV), 0, 0].cpu().numpy().astype(np.complex128))
    assert abs(P[0, 0] - dc) <= 1e-12 * abs(dc)
    del P
    _say("loss path: three pixels against three one-pixel runs")
    m3, _ = dsp.loss(G, k, opt, step=step)
    ms = [dsp.loss(G[j:j + 1].contiguous(), k[j:j + 1], opt, step=step)[0] for j in range(3)]
    want = (ms[0] + ms[1] + ms[2]) / 3.0
    assert float(torch.max(torch.abs(m3 - want))) <= 1e-12
    del G, m3, ms
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [8, 16, 64, 256, 1024])
def test_loss_fused_transform_limits(n):
    """The loss path's fused transforms at their smallest and largest
    power-of-two scans (N = 8 and 1024; other N take hipFFT's transform) and
    at N = 16, 64 and 256, which with the full-frame and the 32 and 128 scans
    of the other loss tests run every pass sequence of the transforms (a
    radix-2 or radix-4 pass first, or radix 8 only) and both column layouts
    (N >= 64 keeps a power-of-two column count per block), three pixels of
    real intensity traces with a bright mean, against the oracle's mean
    phase image and loss."""
    step = 0.373 if n > 8 else 0.9
    opt = _optics(soft=True, det_step=0.02819)
    k = _pixels(opt, 3, 11)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(12 + n)
    G = torch.fft.rfft2(50.0 + torch.randn((3, n, n), generator=gen, device=DEV)).contiguous()
    _say(f"loss at N = {n}: three pixels against the oracle")
    mp, loss = dsp.loss(G, k, opt, step=step)
    torch.cuda.synchronize()
    mp_o, loss_o = O.loss_path(G.cpu().numpy().astype(np.complex128), k, None, n, step, opt)
    assert np.max(np.abs(mp.cpu().numpy() - mp_o)) <= 1e-9
    assert loss == pytest.approx(loss_o, rel=1e-9, abs=1e-15)
    assert np.std(mp_o) > 1e-4
