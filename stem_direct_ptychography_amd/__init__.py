"""Regularized direct (single-side-band) ptychography on MI355X.

Thin Python binding of libdsp.so (include/dsp.h): argument marshalling only.
Every step of the hot path runs in the library's HIP kernels; PyTorch
supplies device memory and the current stream.  There is no CPU fallback:
importing this package raises if the library is missing.

    prep = prepare(G, bf_coords, optics, step=0.373, upsampling=3, method="phase")
    x = prep.solve([1e-2])                  # (S, n_comp, n_q, a_max) complex128
    spec = prep.scatter(x)                  # (S, n_comp, uN, uN/2+1) complex128
    S, N, E = ssb(G, bf_coords, [optics], step=0.373, band=(0.2, 0.9))

``optics`` is any object with attributes ``wavelength``, ``semiangle``,
``det_step``, ``soft``, ``tilt`` (tau_y, tau_x), ``aberrations``
[(n, m, C_nm, phi_nm), ...] and ``depth``, or a dict with those keys.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _lib

_L = _lib.load()

__all__ = ["DspError", "Prepared", "PreparedCache", "prepare", "ssb", "preview", "loss", "quantize_herm16", "geometry_counts", "alias_geometry", "active_bf",
           "band_count", "chi_host", "chi_shift_host", "sincos_host", "LIB_PATH"]

LIB_PATH = _lib.LIB_PATH


class DspError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_lib.STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _check(st: int) -> None:
    if st != _lib.DSP_OK:
        raise DspError(st, _L.dsp_last_error().decode(errors="replace"))


def _get(o, name):
    return o[name] if isinstance(o, dict) else getattr(o, name)


def _optics(o) -> _lib.OpticsC:
    c = _lib.OpticsC()
    c.wavelength_A = float(_get(o, "wavelength"))
    c.semiangle_rad = float(_get(o, "semiangle"))
    c.det_step_invA = float(_get(o, "det_step"))
    c.soft_aperture = 1 if _get(o, "soft") else 0
    t = _get(o, "tilt")
    c.tilt_rad[0] = float(t[0])
    c.tilt_rad[1] = float(t[1])
    c.depth_A = float(_get(o, "depth"))
    ab = list(_get(o, "aberrations"))
    if len(ab) > _lib.MAX_ABERRATIONS:
        raise DspError(_lib.DSP_EINVAL, f"at most {_lib.MAX_ABERRATIONS} aberration terms")
    c.n_aber = len(ab)
    for i, (n, m, cc, phi) in enumerate(ab):
        c.aber[i].n = int(n)
        c.aber[i].m = int(m)
        c.aber[i].c_A = float(cc)
        c.aber[i].phi_rad = float(phi)
    return c


def _dptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _coords(bf_coords) -> np.ndarray:
    k = np.ascontiguousarray(np.asarray(bf_coords, dtype=np.float64))
    if k.ndim != 2 or k.shape[1] != 2:
        raise DspError(_lib.DSP_EINVAL, "bf_coords must be (n_bf, 2) (k_y, k_x)")
    return k


def _weights(weights, n_bf: int) -> Optional[np.ndarray]:
    if weights is None:
        return None
    w = np.ascontiguousarray(np.asarray(weights, dtype=np.float64))
    if w.shape != (n_bf,):
        raise DspError(_lib.DSP_EINVAL, f"weights must be ({n_bf},)")
    return w


def _torch():
    import torch

    return torch


def _check_G(G):
    torch = _torch()
    if not isinstance(G, torch.Tensor) or not G.is_cuda:
        raise DspError(_lib.DSP_EINVAL, "G must be a torch complex64 tensor on the GPU")
    if G.dtype != torch.complex64 or G.dim() != 3 or not G.is_contiguous():
        raise DspError(_lib.DSP_EINVAL, "G must be contiguous complex64 (n_bf, N, N/2+1)")
    n = G.shape[1]
    if G.shape[2] != n // 2 + 1:
        raise DspError(_lib.DSP_EINVAL, f"G's last axis must be N/2+1 = {n // 2 + 1}")
    return n


def _stream(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class Prepared:
    """Prepared per-frequency systems: one reference to a libdsp handle,
    released when the wrapper dies."""

    def __init__(self, handle: ctypes.c_void_p, device, method: str):
        self._h = handle
        self.device = device
        self.method = method
        self.info = self._info()

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _L is not None:   # _L is None at teardown
            _L.dsp_destroy(h)
            self._h = None

    def _info(self) -> dict:
        inf = _lib.InfoC()
        _check(_L.dsp_info(self._h, ctypes.byref(inf)))
        return {
            "n_q": inf.n_q, "a_max": inf.a_max, "n_comp": inf.n_comp, "dim": inf.dim, "n_bf": inf.n_bf,
            "n_active_bf": inf.n_active_bf, "method": inf.method, "upsampling": inf.upsampling,
            "n_scan": inf.n_scan, "n_tiles": inf.n_tiles, "alias_hist": list(inf.alias_hist),
            "scale": inf.scale, "g_bytes": inf.g_bytes, "host_ms": inf.host_ms,
            "layout_ms": inf.layout_ms, "layout_cached": bool(inf.layout_cached),
            "stage_ms": list(inf.stage_ms), "timing_ready": bool(inf.timing_ready), "lobes": inf.lobes,
            "gram": [{"nj": inf.gram_nj[i], "tiles": inf.gram_tiles[i], "waves": inf.gram_waves[i],
                      "ms": inf.gram_ms[i], "fixup_ms": inf.gram_fixup_ms[i],
                      "work": dict(zip(("tests", "lobes", "cols", "pairs", "terms"), list(inf.gram_work[i])))}
                     for i in range(inf.n_gram_launches)],
        }

    def timings(self, stream=None) -> dict:
        """Wait for the prepare's stream, then refresh and return info."""
        torch = _torch()
        s = torch.cuda.current_stream() if stream is None else stream
        s.synchronize()
        self.info = self._info()
        return self.info

    def derive_phase(self, stream=None) -> "Prepared":
        """Phase model from this complex model's systems, with no pass over G
        (dsp_derive_phase)."""
        if self.method != "complex":
            raise ValueError("derive_phase needs a complex-method prepare")
        h = ctypes.c_void_p()
        _check(_L.dsp_derive_phase(self._h, ctypes.c_void_p(_stream(stream)), ctypes.byref(h)))
        return Prepared(h, self.device, "phase")

    def solve(self, strengths, residual: bool = False, stream=None):
        torch = _torch()
        s = np.ascontiguousarray(np.asarray(strengths, dtype=np.float64))
        if self.method == "complex":
            s = s.reshape(-1, 2)
        else:
            s = s.reshape(-1)
        S = s.shape[0]
        inf = self.info
        x = torch.empty((S, inf["n_comp"], inf["n_q"], max(1, inf["a_max"])), dtype=torch.complex128,
                        device=self.device)
        r = torch.empty((S, inf["n_q"]), dtype=torch.float64, device=self.device) if residual else None
        _check(_L.dsp_solve(self._h, _dptr(s), S, ctypes.c_void_p(x.data_ptr()),
                            ctypes.c_void_p(r.data_ptr()) if r is not None else None,
                            ctypes.c_void_p(_stream(stream))))
        return (x, r) if residual else x

    def scatter(self, x, stream=None):
        torch = _torch()
        inf = self.info
        if x.dtype != torch.complex128 or not x.is_contiguous() or x.dim() != 4 or \
                tuple(x.shape[1:]) != (inf["n_comp"], inf["n_q"], max(1, inf["a_max"])):
            raise DspError(_lib.DSP_EINVAL, "x must be the contiguous complex128 output of solve")
        nf = inf["upsampling"] * inf["n_scan"]
        S = x.shape[0]
        spec = torch.empty((S, inf["n_comp"], nf, nf // 2 + 1), dtype=torch.complex128, device=self.device)
        _check(_L.dsp_scatter(self._h, ctypes.c_void_p(x.data_ptr()), S, ctypes.c_void_p(spec.data_ptr()),
                              ctypes.c_void_p(_stream(stream))))
        return spec

    def export_system(self, stream=None):
        """(aug (n_q, D, D) complex128, eig (n_q, a_max) float64 or None)."""
        torch = _torch()
        inf = self.info
        D = inf["dim"]
        aug = torch.empty((inf["n_q"], D, D), dtype=torch.complex128, device=self.device)
        eig = None
        if self.method == "phase":
            eig = torch.empty((inf["n_q"], max(1, inf["a_max"])), dtype=torch.float64, device=self.device)
        _check(_L.dsp_export_system(self._h, ctypes.c_void_p(aug.data_ptr()),
                                    ctypes.c_void_p(eig.data_ptr()) if eig is not None else None,
                                    ctypes.c_void_p(_stream(stream))))
        return aug, eig

    def alias_table(self):
        inf = self.info
        am = max(1, inf["a_max"])
        q = np.zeros((inf["n_q"], 2), dtype=np.int32)
        c = np.zeros(inf["n_q"], dtype=np.int32)
        K = np.zeros((inf["n_q"], am, 2), dtype=np.int32)
        ip = ctypes.POINTER(ctypes.c_int32)
        _check(_L.dsp_alias_table(self._h, q.ctypes.data_as(ip), c.ctypes.data_as(ip), K.ctypes.data_as(ip)))
        return q, c, K


def prepare(G, bf_coords, optics, step: float, upsampling: int, method: str = "phase", weights=None,
            smoothness: float = 0.0, timing: bool = False, count_work: bool = False, slot_test: bool = True,
            stream=None) -> Prepared:
    """Per-frequency normal equations (and, for "phase", the eigenbasis).

    slot_test=False turns off the Gram kernels' per-pixel slot test (every
    alias slot is evaluated at every pixel); the systems do not change."""
    n = _check_G(G)
    k = _coords(bf_coords)
    if k.shape[0] != G.shape[0]:
        raise DspError(_lib.DSP_EINVAL, "bf_coords rows must match G's first axis")
    w = _weights(weights, k.shape[0])
    if method not in ("phase", "complex"):
        raise DspError(_lib.DSP_EINVAL, f"unknown method {method!r}")
    scan = _lib.ScanC(n, float(step))
    flags = ((_lib.DSP_FLAG_TIMING if timing else 0) | (_lib.DSP_FLAG_COUNT_WORK if count_work else 0)
             | (0 if slot_test else _lib.DSP_FLAG_NO_SLOT_TEST))
    opts = _lib.PrepareOptsC(_lib.DSP_PHASE if method == "phase" else _lib.DSP_COMPLEX, int(upsampling),
                             float(smoothness), flags)
    oc = _optics(optics)
    h = ctypes.c_void_p()
    _check(_L.dsp_prepare(ctypes.c_void_p(G.data_ptr()), k.shape[0], _dptr(k), _dptr(w), ctypes.byref(scan),
                          ctypes.byref(oc), ctypes.byref(opts), ctypes.c_void_p(_stream(stream)), ctypes.byref(h)))
    return Prepared(h, G.device, method)


class PreparedCache:
    """Two-slot prepared-model cache (dsp_cache_get): one slot per method
    under the same data and optics key.  Each model it returns holds its own
    reference, so it stays valid after its slot is replaced.

    G is keyed by the tensor itself: the cache keeps a reference to the last
    G it saw and counts a new generation whenever G is a different tensor or
    storage, or its in-place version counter moved, so a new tensor at a
    reused address, or G rewritten in place, is a miss.  The library sees
    that generation times 2^32 plus the caller's own g_version (0 <= g_version
    < 2^32) as its generation number."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(_L.dsp_cache_create(ctypes.byref(h)))
        self._c = h
        self._G = None          # the last G seen (kept alive so its address is not reused)
        self._G_key = None      # (data_ptr, storage ptr, shape, _version)
        self._gen = 0

    def _generation(self, G, g_version: int) -> int:
        if not 0 <= int(g_version) < (1 << 32):
            raise DspError(_lib.DSP_EINVAL, "g_version must be in [0, 2^32)")
        key = (G.data_ptr(), G.untyped_storage().data_ptr(), tuple(G.shape), G._version)
        if self._G is not G or self._G_key != key:
            self._gen += 1
            self._G, self._G_key = G, key
        return (self._gen << 32) | int(g_version)

    def __del__(self):
        c = getattr(self, "_c", None)
        if c and _L is not None:
            _L.dsp_cache_destroy(c)
            self._c = None

    def get(self, G, bf_coords, optics, step: float, upsampling: int, method: str = "phase", weights=None,
            smoothness: float = 0.0, g_version: int = 0, derive: bool = False, stream=None):
        """Returns (Prepared, how) with how "hit", "prepared" or "derived"."""
        n = _check_G(G)
        k = _coords(bf_coords)
        if k.shape[0] != G.shape[0]:
            raise DspError(_lib.DSP_EINVAL, "bf_coords rows must match G's first axis")
        w = _weights(weights, k.shape[0])
        if method not in ("phase", "complex"):
            raise DspError(_lib.DSP_EINVAL, f"unknown method {method!r}")
        scan = _lib.ScanC(n, float(step))
        opts = _lib.PrepareOptsC(_lib.DSP_PHASE if method == "phase" else _lib.DSP_COMPLEX, int(upsampling),
                                 float(smoothness), 0)
        oc = _optics(optics)
        h = ctypes.c_void_p()
        how = ctypes.c_int(-1)
        gen = self._generation(G, g_version)
        _check(_L.dsp_cache_get(self._c, ctypes.c_void_p(G.data_ptr()), gen, k.shape[0], _dptr(k),
                                _dptr(w), ctypes.byref(scan), ctypes.byref(oc), ctypes.byref(opts),
                                1 if derive else 0, ctypes.c_void_p(_stream(stream)), ctypes.byref(h),
                                ctypes.byref(how)))
        return Prepared(h, G.device, method), {0: "prepared", 1: "hit", 2: "derived"}[how.value]


def quantize_herm16(G, rows: bool = False, stream=None):
    """Compact herm16 copy of G (dsp_quantize_herm16): returns (Q int16
    (n_bf, N, N/2+1, 2), scale float32 (n_bf,), or (n_bf, N) with one scale
    per stored row), both on G's device."""
    torch = _torch()
    n = _check_G(G)
    Q = torch.empty(tuple(G.shape) + (2,), dtype=torch.int16, device=G.device)
    sc = torch.empty((G.shape[0], n) if rows else (G.shape[0],), dtype=torch.float32, device=G.device)
    _check(_L.dsp_quantize_herm16(ctypes.c_void_p(G.data_ptr()), G.shape[0], n, 1 if rows else 0,
                                  ctypes.c_void_p(Q.data_ptr()), ctypes.c_void_p(sc.data_ptr()),
                                  ctypes.c_void_p(_stream(stream))))
    return Q, sc


def preview(G, bf_coords, optics, step: float, upsampling: int = 1, weights=None, spectrum: bool = True,
            phase: bool = True, stream=None):
    """Upsampled SSB preview (dsp_preview): returns (P (uN, uN/2+1)
    complex128 or None, phase (uN, uN) float64 or None) on G's device."""
    torch = _torch()
    n = _check_G(G)
    k = _coords(bf_coords)
    if k.shape[0] != G.shape[0]:
        raise DspError(_lib.DSP_EINVAL, "bf_coords rows must match G's first axis")
    w = _weights(weights, k.shape[0])
    m = int(upsampling) * n
    P = torch.empty((m, m // 2 + 1), dtype=torch.complex128, device=G.device) if spectrum else None
    ph = torch.empty((m, m), dtype=torch.float64, device=G.device) if phase else None
    scan = _lib.ScanC(n, float(step))
    _check(_L.dsp_preview(ctypes.c_void_p(G.data_ptr()), k.shape[0], _dptr(k), _dptr(w), ctypes.byref(scan),
                          ctypes.byref(_optics(optics)), int(upsampling),
                          ctypes.c_void_p(P.data_ptr()) if P is not None else None,
                          ctypes.c_void_p(ph.data_ptr()) if ph is not None else None,
                          ctypes.c_void_p(_stream(stream))))
    return P, ph


def loss(G, bf_coords, optics, step: float, weights=None, mean_phase: bool = True, stream=None):
    """Loss path (dsp_loss): returns (mean phase (N, N) float64 on G's device
    or None, loss float)."""
    torch = _torch()
    n = _check_G(G)
    k = _coords(bf_coords)
    if k.shape[0] != G.shape[0]:
        raise DspError(_lib.DSP_EINVAL, "bf_coords rows must match G's first axis")
    w = _weights(weights, k.shape[0])
    mp = torch.empty((n, n), dtype=torch.float64, device=G.device) if mean_phase else None
    out = np.zeros(1, dtype=np.float64)
    scan = _lib.ScanC(n, float(step))
    _check(_L.dsp_loss(ctypes.c_void_p(G.data_ptr()), k.shape[0], _dptr(k), _dptr(w), ctypes.byref(scan),
                       ctypes.byref(_optics(optics)), ctypes.c_void_p(mp.data_ptr()) if mp is not None else None,
                       _dptr(out), ctypes.c_void_p(_stream(stream))))
    return mp, float(out[0])


def _check_Q(Q, scale):
    torch = _torch()
    if not isinstance(Q, torch.Tensor) or not Q.is_cuda or Q.dtype != torch.int16 or Q.dim() != 4 \
            or Q.shape[3] != 2 or not Q.is_contiguous():
        raise DspError(_lib.DSP_EINVAL, "Q must be contiguous int16 (n_bf, N, N/2+1, 2) on the GPU")
    n = Q.shape[1]
    if Q.shape[2] != n // 2 + 1:
        raise DspError(_lib.DSP_EINVAL, f"Q's third axis must be N/2+1 = {n // 2 + 1}")
    if not isinstance(scale, torch.Tensor) or scale.dtype != torch.float32 or scale.device != Q.device \
            or tuple(scale.shape) not in ((Q.shape[0],), (Q.shape[0], n)) or not scale.is_contiguous():
        raise DspError(_lib.DSP_EINVAL, "scale must be contiguous float32 (n_bf,) or (n_bf, N) on Q's device")
    return n


def ssb(G, bf_coords, optics_sets: Sequence, step: float, band: Optional[Tuple[float, float]] = None,
        weights=None, want_S: bool = True, want_N: bool = True, agreement: bool = True, stream=None,
        herm16=None, no_alloc: bool = False, out=None):
    """SSB sums for up to 8 optics sets in one pass over G.

    ``herm16=(Q, scale)`` from quantize_herm16 runs the pass over the compact
    copy instead (G may then be None).  ``no_alloc=True`` runs the
    allocation-free pass (dsp_ssb_noalloc: the library allocates no device
    memory); with ``out=(S, N)`` (either may be None) the outputs are written
    into those tensors instead of new ones.  Returns (S (B, N, N/2+1)
    complex128 or None, N (B, N, N/2+1) float64 or None, E (B,) numpy float64
    or None)."""
    torch = _torch()
    if no_alloc and herm16 is not None:
        raise DspError(_lib.DSP_EINVAL, "the allocation-free pass reads complex64 G")
    if herm16 is not None:
        Q, sc = herm16
        n = _check_Q(Q, sc)
        n_rows, device = Q.shape[0], Q.device
    else:
        n = _check_G(G)
        n_rows, device = G.shape[0], G.device
    k = _coords(bf_coords)
    if k.shape[0] != n_rows:
        raise DspError(_lib.DSP_EINVAL, "bf_coords rows must match G's first axis")
    w = _weights(weights, k.shape[0])
    B = len(optics_sets)
    arr = (_lib.OpticsC * max(1, B))()
    for i, o in enumerate(optics_sets):
        arr[i] = _optics(o)
    scan = _lib.ScanC(n, float(step))
    nh = n // 2 + 1
    if out is not None:
        S, Nn = out
        for t, dt in ((S, torch.complex128), (Nn, torch.float64)):
            if t is not None and (t.dtype != dt or tuple(t.shape) != (B, n, nh) or not t.is_contiguous()
                                  or t.device != device):
                raise DspError(_lib.DSP_EINVAL, f"out tensors must be contiguous {(B, n, nh)} on {device}")
    else:
        S = torch.empty((B, n, nh), dtype=torch.complex128, device=device) if want_S else None
        Nn = torch.empty((B, n, nh), dtype=torch.float64, device=device) if want_N else None
    E = np.zeros(max(1, B), dtype=np.float64) if agreement else None
    bd = np.asarray(band, dtype=np.float64) if band is not None else None
    outs = (_dptr(bd), ctypes.c_void_p(S.data_ptr()) if S is not None else None,
            ctypes.c_void_p(Nn.data_ptr()) if Nn is not None else None, _dptr(E) if E is not None else None,
            ctypes.c_void_p(_stream(stream)))
    if herm16 is not None:
        _check(_L.dsp_ssb_herm16(ctypes.c_void_p(Q.data_ptr()), ctypes.c_void_p(sc.data_ptr()),
                                 1 if sc.dim() == 2 else 0, k.shape[0], _dptr(k), _dptr(w), ctypes.byref(scan), arr,
                                 B, *outs))
    else:
        fn = _L.dsp_ssb_noalloc if no_alloc else _L.dsp_ssb
        _check(fn(ctypes.c_void_p(G.data_ptr()), k.shape[0], _dptr(k), _dptr(w), ctypes.byref(scan), arr, B, *outs))
    return S, Nn, (E[:B] if E is not None else None)


# ---------------------------------------------------------------------------
# host-only geometry (no device calls)
# ---------------------------------------------------------------------------


def geometry_counts(n_scan: int, step: float, optics, upsampling: int):
    """(n_q, a_max, alias histogram[10]) computed by the library's host code."""
    scan = _lib.ScanC(int(n_scan), float(step))
    oc = _optics(optics)
    nq, am = ctypes.c_int(), ctypes.c_int()
    hist = np.zeros(10, dtype=np.int32)
    _check(_L.dsp_geometry_counts(ctypes.byref(scan), ctypes.byref(oc), int(upsampling), ctypes.byref(nq),
                                  ctypes.byref(am), hist.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return nq.value, am.value, hist


def alias_geometry(n_scan: int, step: float, optics, upsampling: int):
    """(q (n_q, 2), count (n_q,), K (n_q, a_max, 2)) int32 from the library's host code."""
    nq, am, _ = geometry_counts(n_scan, step, optics, upsampling)
    scan = _lib.ScanC(int(n_scan), float(step))
    oc = _optics(optics)
    q = np.zeros((nq, 2), dtype=np.int32)
    c = np.zeros(nq, dtype=np.int32)
    K = np.zeros((nq, max(1, am), 2), dtype=np.int32)
    ip = ctypes.POINTER(ctypes.c_int32)
    _check(_L.dsp_alias_geometry(ctypes.byref(scan), ctypes.byref(oc), int(upsampling), q.ctypes.data_as(ip),
                                 c.ctypes.data_as(ip), K.ctypes.data_as(ip)))
    return q, c, K


def active_bf(bf_coords, optics) -> np.ndarray:
    k = _coords(bf_coords)
    idx = np.zeros(k.shape[0], dtype=np.int32)
    n = ctypes.c_int()
    _check(_L.dsp_active_bf(_dptr(k), k.shape[0], ctypes.byref(_optics(optics)),
                            idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(n)))
    return idx[: n.value]


def band_count(n_scan: int, step: float, band) -> int:
    scan = _lib.ScanC(int(n_scan), float(step))
    bd = np.asarray(band, dtype=np.float64) if band is not None else None
    n = ctypes.c_int()
    _check(_L.dsp_band_count(ctypes.byref(scan), _dptr(bd), ctypes.byref(n)))
    return n.value


def sincos_host(x) -> Tuple[np.ndarray, np.ndarray]:
    """The library's FP64 sine and cosine (the kernels' source) on the host."""
    xx = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1))
    s = np.zeros_like(xx)
    c = np.zeros_like(xx)
    _check(_L.dsp_sincos_host(_dptr(xx), xx.shape[0], _dptr(s), _dptr(c)))
    return s, c


def atan2_host(y, x) -> np.ndarray:
    """The loss path's FP64 atan2 (the kernels' source) on the host."""
    yy = np.ascontiguousarray(np.asarray(y, dtype=np.float64).reshape(-1))
    xx = np.ascontiguousarray(np.broadcast_to(np.asarray(x, dtype=np.float64), yy.shape).reshape(-1))
    out = np.zeros_like(yy)
    _check(_L.dsp_atan2_host(_dptr(yy), _dptr(xx), yy.shape[0], _dptr(out)))
    return out


def chi_host(optics, k) -> np.ndarray:
    """The library's aberration polynomial chi(k) evaluated on the host."""
    kk = _coords(k)
    out = np.zeros(kk.shape[0], dtype=np.float64)
    _check(_L.dsp_chi_host(ctypes.byref(_optics(optics)), _dptr(kk), kk.shape[0], _dptr(out)))
    return out


def chi_shift_host(optics, k, Q) -> np.ndarray:
    """The lobes' phase differences as the Gram kernels form them, on the
    host: (n, 2) of (chi(k - Q) - chi(k), chi(k + Q) - chi(k))."""
    kk = _coords(k)
    qq = _coords(Q)
    if qq.shape != kk.shape:
        raise DspError(_lib.DSP_EINVAL, "k and Q must have the same shape")
    out = np.zeros((kk.shape[0], 2), dtype=np.float64)
    _check(_L.dsp_chi_shift_host(ctypes.byref(_optics(optics)), _dptr(kk), _dptr(qq), kk.shape[0], _dptr(out)))
    return out
