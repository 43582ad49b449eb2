"""The allocation-free SSB pass (dsp_ssb_noalloc) through the C ABI, against
dsp_ssb on the same inputs.

Both passes compute the same sums; the allocation-free one may cut each
frequency's pixel sum into fewer stream-K pieces (its plan is sized to the
fixed scratch), so the results agree to rounding: the parity bar of the SSB
pass, 1e-5 relative globally and per entry, and 1e-6 on the agreement.  The
calls run back to back, each later one on a smaller input than the one
before, so stale scratch contents would show.  The device's free memory is
read around each call: the call allocates nothing.
"""
import ctypes

import numpy as np
import pytest

from oracle import dsp_oracle as O
from synthetic import bf_pixels, data_stack_numpy, data_stack_torch, ssb_sets, workload

torch = pytest.importorskip("torch")
dsp = pytest.importorskip("stem_direct_ptychography_amd")
from stem_direct_ptychography_amd import _lib  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-5


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)


def _noalloc(G, k, sets, step, band, S, Nn):
    """dsp_ssb_noalloc through ctypes into preallocated S, N; returns
    (status, agreement)."""
    L = dsp._L
    kk = np.ascontiguousarray(k, dtype=np.float64)
    B = len(sets)
    arr = (_lib.OpticsC * B)()
    for i, o in enumerate(sets):
        arr[i] = dsp._optics(o)
    scan = _lib.ScanC(G.shape[1], float(step))
    bd = None if band is None else np.asarray(band, dtype=np.float64)
    E = np.zeros(B)
    dp = ctypes.POINTER(ctypes.c_double)
    st = L.dsp_ssb_noalloc(ctypes.c_void_p(G.data_ptr()), kk.shape[0], kk.ctypes.data_as(dp), None,
                           ctypes.byref(scan), arr, B, None if bd is None else bd.ctypes.data_as(dp),
                           ctypes.c_void_p(S.data_ptr()), ctypes.c_void_p(Nn.data_ptr()), E.ctypes.data_as(dp),
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, E


def _compare(name, G, k, sets, step, band):
    B = len(sets)
    n = G.shape[1]
    S_ref, N_ref, E_ref = dsp.ssb(G, k, sets, step=step, band=band)
    S = torch.full((B, n, n // 2 + 1), complex(7.0, 7.0), dtype=torch.complex128, device=DEV)
    Nn = torch.full((B, n, n // 2 + 1), 7.0, dtype=torch.float64, device=DEV)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    _say(f"{name}: B={B} N={n} n_bf={len(k)} band={band}")
    st, E = _noalloc(G, k, sets, step, band, S, Nn)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert st == _lib.DSP_OK, dsp._L.dsp_last_error().decode()
    assert free1 == free0, f"{name}: device free memory moved by {free0 - free1} bytes"
    for b in range(B):
        ref, got = S_ref[b], S[b]
        glob = (torch.linalg.norm(got - ref) / torch.linalg.norm(ref)).item()
        den = torch.clamp(ref.abs(), min=1e-3 * ref.abs().max().item())
        loc = ((got - ref).abs() / den).max().item()
        assert glob <= TOL and loc <= TOL, f"{name} set {b}: S {glob:.2e} {loc:.2e}"
        nr, ng = N_ref[b], Nn[b]
        nden = torch.clamp(nr.abs(), min=1e-3 * nr.abs().max().item())
        assert ((ng - nr).abs() / nden).max().item() <= TOL, f"{name} set {b}: N"
    # outside the band both write zeros (the sentinel 7 is gone everywhere)
    if band is not None:
        mask = torch.as_tensor(O.band_mask(n, step, band), device=DEV)
        assert not torch.any(S[:, ~mask]) and not torch.any(Nn[:, ~mask])
    assert np.allclose(E, E_ref, rtol=1e-6, atol=0), (E, E_ref)
    _say(f"{name}: agrees with dsp_ssb, agreement {E}")


def test_noalloc_matches_ssb_on_shrinking_inputs():
    """Full-frame band pass (8 sets), then the 128 x 128 scan's whole plane
    (3 sets), then the tiny 32 x 32 scan (1 set): each against dsp_ssb."""
    w5 = workload("c5")
    pix, k5 = bf_pixels(w5)
    _say("generating the agreement-pass G (8807, 512, 257) on the GPU")
    G5 = data_stack_torch(w5, pix, DEV)
    torch.cuda.synchronize()
    _compare("full frame", G5, k5, ssb_sets(w5, 8), w5.step, w5.band)
    del G5
    torch.cuda.empty_cache()
    w2 = workload("c2")
    pix, k2 = bf_pixels(w2)
    G2 = torch.as_tensor(data_stack_numpy(w2, pix), device=DEV)
    sets2 = [w2.optics, w2.optics.replace(tilt=(1e-3, 0.0)), w2.optics.replace(depth=60.0)]
    _compare("128 x 128", G2, k2, sets2, w2.step, None)
    w1 = workload("c1")
    pix, k1 = bf_pixels(w1)
    G1 = torch.as_tensor(data_stack_numpy(w1, pix), device=DEV)
    _compare("32 x 32", G1, k1, [w1.optics], w1.step, (0.1, 2.9))
    # and the larger one again after the smaller
    _compare("128 x 128 again", G2, k2, sets2[:2], w2.step, (0.2, 1.5))


def test_noalloc_frees_nothing_with_full_layout_caches():
    """After more allocating passes than the layout caches hold (each band a
    new layout), allocation-free passes with new bands evict no layout that
    holds device memory: the device's free memory does not move and the sums
    match dsp_ssb."""
    w1 = workload("c1")
    pix, k1 = bf_pixels(w1)
    G1 = torch.as_tensor(data_stack_numpy(w1, pix), device=DEV)
    for i in range(6):
        dsp.ssb(G1, k1, [w1.optics], step=w1.step, band=(0.1 + 0.05 * i, 2.9))
    torch.cuda.synchronize()
    for i in range(6):
        _compare(f"32 x 32 band {i}", G1, k1, [w1.optics], w1.step, (0.12 + 0.05 * i, 2.8))


def test_noalloc_rejects_a_pass_beyond_its_scratch():
    """A pass whose tables alone exceed the fixed scratch (8 sets over 60,000
    pixels: 8 x 60,000 x 160 bytes of Taylor tables) returns DSP_ENOMEM with a
    message before any device work; dsp_ssb itself runs it."""
    w = workload("c1")
    rng = np.random.default_rng(3)
    n_bf = 60000
    kc = w.optics.semiangle / w.optics.wavelength
    r = np.sqrt(rng.uniform(0, 1, n_bf)) * 0.9 * kc
    t = rng.uniform(0, 2 * np.pi, n_bf)
    k = np.stack([r * np.sin(t), r * np.cos(t)], axis=1)
    G = torch.zeros((n_bf, w.n_scan, w.n_half), dtype=torch.complex64, device=DEV)
    B = 8
    sets = [w.optics.replace(aberrations=[(1, 0, -100.0 + 5 * b, 0.0)]) for b in range(B)]
    S = torch.zeros((B, w.n_scan, w.n_half), dtype=torch.complex128, device=DEV)
    Nn = torch.zeros((B, w.n_scan, w.n_half), dtype=torch.float64, device=DEV)
    torch.cuda.synchronize()
    st, _ = _noalloc(G, k, sets, w.step, (0.1, 2.9), S, Nn)
    msg = dsp._L.dsp_last_error().decode()
    assert st == _lib.DSP_ENOMEM and "scratch" in msg, (st, msg)
    assert not torch.any(S) and not torch.any(Nn)
    Sr, Nr, Er = dsp.ssb(G, k, sets, step=w.step, band=(0.1, 2.9))
    torch.cuda.synchronize()
    assert not torch.any(Sr)
