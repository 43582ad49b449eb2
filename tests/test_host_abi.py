"""Host logic of libdsp, checked on the CPU through its C ABI.

No device calls: the library loads without a GPU, its host geometry is
compared bit for bit with the oracle's independent implementation, and its
argument validation returns the documented status codes.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from oracle import dsp_oracle as O
from synthetic import LAMBDA_300KV, Optics, bf_pixels, random_weights, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

dsp = pytest.importorskip("stem_direct_ptychography_amd")
from stem_direct_ptychography_amd import _lib  # noqa: E402


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "dsp.h")).read()
    declared = set(re.findall(r"\b(dsp_[a-z0-9_]+)\s*\(", hdr))
    assert declared, "no declarations parsed"
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(_lib.EXPORTS)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_alias_geometry_bit_exact(name):
    w = workload(name)
    q, counts, Ks = O.alias_table(w.n_scan, w.step, w.upsampling, w.optics)
    nq, am, hist = dsp.geometry_counts(w.n_scan, w.step, w.optics, w.upsampling)
    assert nq == len(q)
    assert am == counts.max()
    want = np.bincount(counts, minlength=10)
    assert np.array_equal(hist, want)
    ql, cl, Kl = dsp.alias_geometry(w.n_scan, w.step, w.optics, w.upsampling)
    assert np.array_equal(ql, q)
    assert np.array_equal(cl, counts)
    for i in range(0, len(q), max(1, len(q) // 5000)):
        A = counts[i]
        assert np.array_equal(Kl[i, :A], Ks[i])
        assert not Kl[i, A:].any()


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_active_set_bit_exact(name):
    w = workload(name)
    _, k = bf_pixels(w)
    assert np.array_equal(dsp.active_bf(k, w.optics), O.active_pixels(k, w.optics))
    # a disk larger than the aperture: the edge pixels drop out identically
    k2 = k * 1.3
    assert np.array_equal(dsp.active_bf(k2, w.optics), O.active_pixels(k2, w.optics))


def test_band_count_bit_exact():
    w = workload("c5")
    assert dsp.band_count(w.n_scan, w.step, w.band) == int(O.band_mask(w.n_scan, w.step, w.band).sum())
    assert dsp.band_count(64, 0.5, None) == 64 * 33


@pytest.mark.parametrize("name", ["c2", "c3"])
def test_chi_polynomial_matches_oracle(name):
    w = workload(name)
    rng = np.random.default_rng(0)
    kc = w.optics.semiangle / w.optics.wavelength
    k = rng.uniform(-2.2 * kc, 2.2 * kc, size=(2000, 2))
    got = dsp.chi_host(w.optics, k)
    want = O.chi(k[:, 0], k[:, 1], w.optics)
    assert np.max(np.abs(got - want)) <= 1e-11 * max(1.0, np.max(np.abs(want)))


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_chi_shift_matches_oracle(name):
    """The Gram kernels' lobe phases (chi expanded about theta(k), even and
    odd parts in lambda Q) against the oracle's chi differences, pixels in
    the aperture and frequencies out to the alias radius."""
    w = workload(name)
    rng = np.random.default_rng(2)
    kc = w.optics.semiangle / w.optics.wavelength
    k = rng.uniform(-1.05 * kc, 1.05 * kc, size=(3000, 2))
    Q = rng.uniform(-2.1 * kc, 2.1 * kc, size=(3000, 2))
    Q[:5] = 0.0
    got = dsp.chi_shift_host(w.optics, k, Q)
    c0 = O.chi(k[:, 0], k[:, 1], w.optics)
    want_l = O.chi(k[:, 0] - Q[:, 0], k[:, 1] - Q[:, 1], w.optics) - c0
    want_r = O.chi(k[:, 0] + Q[:, 0], k[:, 1] + Q[:, 1], w.optics) - c0
    scale = max(1.0, np.max(np.abs(c0)), np.max(np.abs(want_l)), np.max(np.abs(want_r)))
    assert np.max(np.abs(got[:, 0] - want_l)) <= 1e-11 * scale
    assert np.max(np.abs(got[:, 1] - want_r)) <= 1e-11 * scale
    assert not np.any(got[:5])   # Q = 0: no phase difference, exactly


def test_chi_polynomial_every_term():
    rng = np.random.default_rng(1)
    k = rng.uniform(-3.0, 3.0, size=(200, 2))
    for n, m in [(1, 0), (1, 2), (2, 1), (2, 3), (3, 0), (3, 2), (3, 4), (4, 1), (4, 3), (4, 5),
                 (5, 0), (5, 2), (5, 4), (5, 6)]:
        o = Optics(LAMBDA_300KV, 0.03, 0.03, tilt=(1e-3, -2e-3), aberrations=[(n, m, 1.0e3 * n, 0.37 * m)])
        got = dsp.chi_host(o, k)
        want = O.chi(k[:, 0], k[:, 1], o)
        assert np.max(np.abs(got - want)) <= 1e-11 * max(1.0, np.max(np.abs(want))), (n, m)


def test_sincos_matches_libm():
    """The kernels' FP64 sine/cosine against the C library's, over the phase
    range the transfer produces and at the quadrant boundaries."""
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.uniform(-400.0, 400.0, 200000), rng.uniform(-1.0, 1.0, 20000),
                        np.arange(-64, 65) * (math.pi / 4), np.arange(-64, 65) * (math.pi / 4) + 1e-12,
                        np.arange(-64, 65) * (math.pi / 4) - 1e-12, [0.0, -0.0, 1e-300, -1e-300, 5e-324]])
    s, c = dsp.sincos_host(x)
    # the method's bound: the sine's truncation r^5/120 at |r| = pi/256 is
    # 2.4e-12 (the angle addition carries it into both outputs), the
    # cosine's r^6/720 below 5e-15; the reduction constant adds 4e-17 |x|
    # (1.6e-14 at |x| = 400); plus rounding
    red = 4e-17 * np.max(np.abs(x))
    bound = (math.pi / 256) ** 5 / 120 + red + 1e-15
    assert np.max(np.abs(s - np.sin(x))) <= bound
    assert np.max(np.abs(c - np.cos(x))) <= bound
    assert np.max(np.abs(s * s + c * c - 1.0)) <= 2 * bound


def test_atan2_matches_libm():
    """The loss path's table-reduced atan2 against the C library's: both
    signs of x (x < 0 takes the +-pi branch), |y/x| across 16 decades, the
    fold at |y/x| = 1, the table's nodes i/64 and the signed zeros."""
    rng = np.random.default_rng(3)
    n = 200000
    y = rng.standard_normal(n) * np.exp(rng.uniform(-18.0, 18.0, n))
    x = rng.choice([1.0, -1.0, 37.5, -0.01, 2.5e4], n)
    nodes = np.arange(65) / 64.0
    y = np.concatenate([y, nodes, -nodes, nodes + 1e-9, 1.0 / np.maximum(nodes, 1e-3), [0.0, -0.0, 0.0, -0.0, 1.0]])
    x = np.concatenate([x, np.ones(65), -np.ones(65), np.ones(65), np.ones(65), [1.0, 1.0, -1.0, -1.0, 0.0]])
    got = dsp.atan2_host(y, x)
    ref = np.arctan2(y, x)
    # 3 ulp of the result: the reduction's rounding and t = y (1/x)
    assert np.all(np.abs(got - ref) <= 3 * np.spacing(np.abs(ref)) + 1e-300)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def _status(fn, *args):
    return fn(*args)


def test_validation_status_codes():
    w = workload("c2")
    good = _lib.ScanC(128, 0.4)
    oc = dsp._optics(w.optics)
    nq, am = ctypes.c_int(), ctypes.c_int()
    L = dsp._L
    assert L.dsp_geometry_counts(ctypes.byref(good), ctypes.byref(oc), 2, ctypes.byref(nq), ctypes.byref(am),
                                 None) == _lib.DSP_OK
    odd = _lib.ScanC(127, 0.4)
    assert L.dsp_geometry_counts(ctypes.byref(odd), ctypes.byref(oc), 2, None, None, None) == _lib.DSP_EUNSUPPORTED
    bad_step = _lib.ScanC(128, -1.0)
    assert L.dsp_geometry_counts(ctypes.byref(bad_step), ctypes.byref(oc), 2, None, None, None) == _lib.DSP_EINVAL
    assert L.dsp_geometry_counts(ctypes.byref(good), ctypes.byref(oc), 5, None, None, None) == _lib.DSP_EUNSUPPORTED
    assert L.dsp_geometry_counts(ctypes.byref(good), ctypes.byref(oc), 0, None, None, None) == _lib.DSP_EINVAL
    deep = dsp._optics(w.optics.replace(depth=124.0))
    assert L.dsp_geometry_counts(ctypes.byref(good), ctypes.byref(deep), 2, None, None, None) == _lib.DSP_OK
    for bad_depth in (-1.0, float("nan"), float("inf")):
        o = dsp._optics(w.optics.replace(depth=bad_depth))
        assert L.dsp_geometry_counts(ctypes.byref(good), ctypes.byref(o), 2, None, None, None) == _lib.DSP_EINVAL
    bad_ab = dsp._optics(w.optics.replace(aberrations=[(1, 1, 10.0, 0.0)]))
    assert L.dsp_geometry_counts(ctypes.byref(good), ctypes.byref(bad_ab), 2, None, None, None) == _lib.DSP_EINVAL
    assert "Krivanek" in L.dsp_last_error().decode()
    neg = dsp._optics(w.optics.replace(wavelength=0.0))
    assert L.dsp_geometry_counts(ctypes.byref(good), ctypes.byref(neg), 2, None, None, None) == _lib.DSP_EINVAL
    # prepare / ssb reject bad arguments before touching the device
    _, k = bf_pixels(w)
    k = np.ascontiguousarray(k)
    kp = k.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    opts = _lib.PrepareOptsC(0, 2, 0.0, 0)
    h = ctypes.c_void_p()
    assert L.dsp_prepare(None, len(k), kp, None, ctypes.byref(good), ctypes.byref(oc), ctypes.byref(opts), None,
                         ctypes.byref(h)) == _lib.DSP_EINVAL
    fake = ctypes.c_void_p(0x1000)
    bad_opts = _lib.PrepareOptsC(7, 2, 0.0, 0)
    assert L.dsp_prepare(fake, len(k), kp, None, ctypes.byref(good), ctypes.byref(oc), ctypes.byref(bad_opts), None,
                         ctypes.byref(h)) == _lib.DSP_EINVAL
    assert L.dsp_prepare(fake, 0, kp, None, ctypes.byref(good), ctypes.byref(oc), ctypes.byref(opts), None,
                         ctypes.byref(h)) == _lib.DSP_EINVAL
    bad_flags = _lib.PrepareOptsC(0, 2, 0.0, 8)
    assert L.dsp_prepare(fake, len(k), kp, None, ctypes.byref(good), ctypes.byref(oc), ctypes.byref(bad_flags), None,
                         ctypes.byref(h)) == _lib.DSP_EINVAL
    assert "flags" in L.dsp_last_error().decode()
    wneg = -np.ones(len(k))
    assert L.dsp_prepare(fake, len(k), kp, wneg.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), ctypes.byref(good),
                         ctypes.byref(oc), ctypes.byref(opts), None, ctypes.byref(h)) == _lib.DSP_EINVAL
    arr = (_lib.OpticsC * 2)(oc, dsp._optics(w.optics.replace(semiangle=0.02)))
    assert L.dsp_ssb(fake, len(k), kp, None, ctypes.byref(good), arr, 2, None, None, None, None,
                     None) == _lib.DSP_EINVAL
    assert L.dsp_ssb(fake, len(k), kp, None, ctypes.byref(good), arr, 9, None, None, None, None,
                     None) == _lib.DSP_EINVAL
    assert L.dsp_solve(None, None, 1, None, None, None) == _lib.DSP_EINVAL
    # prepared-model cache: argument checks need no device
    cache = ctypes.c_void_p()
    assert L.dsp_cache_create(None) == _lib.DSP_EINVAL
    assert L.dsp_cache_create(ctypes.byref(cache)) == _lib.DSP_OK and cache.value
    hh = ctypes.c_void_p()
    assert L.dsp_cache_get(None, fake, 0, len(k), kp, None, ctypes.byref(good), ctypes.byref(oc), ctypes.byref(opts),
                           0, None, ctypes.byref(hh), None) == _lib.DSP_EINVAL
    assert L.dsp_cache_get(cache, fake, 0, len(k), kp, None, ctypes.byref(good), ctypes.byref(oc),
                           ctypes.byref(bad_opts), 0, None, ctypes.byref(hh), None) == _lib.DSP_EINVAL
    L.dsp_cache_destroy(cache)
    # herm16: null buffers, bad sizes (caught before any device call)
    assert L.dsp_quantize_herm16(None, 4, 16, 0, None, None, None) == _lib.DSP_EINVAL
    assert L.dsp_quantize_herm16(ctypes.c_void_p(16), 0, 16, 1, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                 None) == _lib.DSP_EINVAL
    assert L.dsp_quantize_herm16(ctypes.c_void_p(16), 4, 15, 0, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                 None) == _lib.DSP_EINVAL
    assert L.dsp_ssb_herm16(None, None, 0, 1, None, None, ctypes.byref(good), ctypes.byref(oc), 1, None, None, None,
                            None, None) == _lib.DSP_EINVAL
    assert L.dsp_info(None, None) == _lib.DSP_EINVAL


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    w = workload("c1")
    _, k = bf_pixels(w)
    G = torch.zeros((len(k), 32, 17), dtype=torch.complex64)
    with pytest.raises(dsp.DspError):
        dsp.prepare(G, k, w.optics, step=w.step, upsampling=1)


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: any --gpus other than 1 exits with status 2
    and a message before touching a device."""
    import subprocess
    import sys as _sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([_sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout.strip() == ""
