"""ctypes declarations of libdsp.so (mirrors include/dsp.h).

Loading fails loudly: there is no CPU fallback for any entry point.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsp.so")

DSP_OK, DSP_EINVAL, DSP_EUNSUPPORTED, DSP_EALIAS, DSP_ENOMEM, DSP_EDEVICE = range(6)
STATUS_NAMES = {0: "DSP_OK", 1: "DSP_EINVAL", 2: "DSP_EUNSUPPORTED", 3: "DSP_EALIAS", 4: "DSP_ENOMEM",
                5: "DSP_EDEVICE"}
DSP_PHASE, DSP_COMPLEX = 0, 1
DSP_FLAG_TIMING = 1
DSP_FLAG_COUNT_WORK = 2
DSP_FLAG_NO_SLOT_TEST = 4
MAX_ABERRATIONS = 16


class Aberration(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int), ("m", ctypes.c_int), ("c_A", ctypes.c_double), ("phi_rad", ctypes.c_double)]


class OpticsC(ctypes.Structure):
    _fields_ = [
        ("wavelength_A", ctypes.c_double),
        ("semiangle_rad", ctypes.c_double),
        ("det_step_invA", ctypes.c_double),
        ("soft_aperture", ctypes.c_int),
        ("tilt_rad", ctypes.c_double * 2),
        ("depth_A", ctypes.c_double),
        ("n_aber", ctypes.c_int),
        ("aber", Aberration * MAX_ABERRATIONS),
    ]


class ScanC(ctypes.Structure):
    _fields_ = [("n_scan", ctypes.c_int), ("step_A", ctypes.c_double)]


class PrepareOptsC(ctypes.Structure):
    _fields_ = [("method", ctypes.c_int), ("upsampling", ctypes.c_int), ("smoothness_invA", ctypes.c_double),
                ("flags", ctypes.c_int)]


class InfoC(ctypes.Structure):
    _fields_ = [
        ("n_q", ctypes.c_int), ("a_max", ctypes.c_int), ("n_comp", ctypes.c_int), ("dim", ctypes.c_int),
        ("n_bf", ctypes.c_int), ("n_active_bf", ctypes.c_int), ("method", ctypes.c_int),
        ("upsampling", ctypes.c_int), ("n_scan", ctypes.c_int), ("n_tiles", ctypes.c_int),
        ("alias_hist", ctypes.c_int * 10), ("scale", ctypes.c_double), ("g_bytes", ctypes.c_double),
        ("lobes", ctypes.c_double), ("host_ms", ctypes.c_double), ("layout_ms", ctypes.c_double),
        ("layout_cached", ctypes.c_int), ("stage_ms", ctypes.c_double * 4),
        ("timing_ready", ctypes.c_int),
        ("n_gram_launches", ctypes.c_int), ("gram_nj", ctypes.c_int * 16), ("gram_tiles", ctypes.c_int * 16),
        ("gram_waves", ctypes.c_int * 16), ("gram_ms", ctypes.c_double * 16), ("gram_fixup_ms", ctypes.c_double * 16), ("gram_work", (ctypes.c_double * 5) * 16),
    ]


# every symbol include/dsp.h declares
EXPORTS = (
    "dsp_prepare", "dsp_solve", "dsp_scatter", "dsp_ssb", "dsp_info", "dsp_export_system", "dsp_alias_table",
    "dsp_destroy", "dsp_last_error", "dsp_geometry_counts", "dsp_alias_geometry", "dsp_active_bf",
    "dsp_band_count", "dsp_chi_host", "dsp_chi_shift_host", "dsp_sincos_host", "dsp_atan2_host", "dsp_derive_phase", "dsp_quantize_herm16",
    "dsp_ssb_herm16", "dsp_preview", "dsp_loss", "dsp_cache_create", "dsp_cache_destroy", "dsp_cache_get",
    "dsp_ssb_noalloc",
)

NOALLOC_SCRATCH_BYTES = 64 << 20   # DSP_NOALLOC_SCRATCH_BYTES

_P = ctypes.c_void_p
_I = ctypes.c_int
_DP = ctypes.POINTER(ctypes.c_double)
_IP = ctypes.POINTER(ctypes.c_int32)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"libdsp.so not found at {path}; build it with `python -m stem_direct_ptychography_amd.build` "
            "(hipcc, gfx950).  There is no CPU fallback.")
    lib = ctypes.CDLL(path)
    for name in EXPORTS:
        if not hasattr(lib, name):
            raise ImportError(f"{path} does not export {name}")
    lib.dsp_last_error.restype = ctypes.c_char_p
    lib.dsp_last_error.argtypes = []
    lib.dsp_destroy.restype = None
    lib.dsp_destroy.argtypes = [_P]
    lib.dsp_prepare.restype = _I
    lib.dsp_prepare.argtypes = [_P, _I, _DP, _DP, ctypes.POINTER(ScanC), ctypes.POINTER(OpticsC),
                                ctypes.POINTER(PrepareOptsC), _P, ctypes.POINTER(_P)]
    lib.dsp_derive_phase.restype = _I
    lib.dsp_derive_phase.argtypes = [_P, _P, ctypes.POINTER(_P)]
    lib.dsp_solve.restype = _I
    lib.dsp_solve.argtypes = [_P, _DP, _I, _P, _P, _P]
    lib.dsp_scatter.restype = _I
    lib.dsp_scatter.argtypes = [_P, _P, _I, _P, _P]
    lib.dsp_ssb.restype = _I
    lib.dsp_ssb.argtypes = [_P, _I, _DP, _DP, ctypes.POINTER(ScanC), ctypes.POINTER(OpticsC), _I, _DP, _P, _P,
                            _DP, _P]
    lib.dsp_ssb_noalloc.restype = _I
    lib.dsp_ssb_noalloc.argtypes = [_P, _I, _DP, _DP, ctypes.POINTER(ScanC), ctypes.POINTER(OpticsC), _I, _DP, _P,
                                    _P, _DP, _P]
    lib.dsp_ssb_herm16.restype = _I
    lib.dsp_ssb_herm16.argtypes = [_P, _P, _I, _I, _DP, _DP, ctypes.POINTER(ScanC), ctypes.POINTER(OpticsC), _I,
                                   _DP, _P, _P, _DP, _P]
    lib.dsp_preview.restype = _I
    lib.dsp_preview.argtypes = [_P, _I, _DP, _DP, ctypes.POINTER(ScanC), ctypes.POINTER(OpticsC), _I, _P, _P, _P]
    lib.dsp_cache_create.restype = _I
    lib.dsp_cache_create.argtypes = [ctypes.POINTER(_P)]
    lib.dsp_cache_destroy.restype = None
    lib.dsp_cache_destroy.argtypes = [_P]
    lib.dsp_cache_get.restype = _I
    lib.dsp_cache_get.argtypes = [_P, _P, ctypes.c_ulonglong, _I, _DP, _DP, ctypes.POINTER(ScanC),
                                  ctypes.POINTER(OpticsC), ctypes.POINTER(PrepareOptsC), _I, _P, ctypes.POINTER(_P),
                                  ctypes.POINTER(_I)]
    lib.dsp_loss.restype = _I
    lib.dsp_loss.argtypes = [_P, _I, _DP, _DP, ctypes.POINTER(ScanC), ctypes.POINTER(OpticsC), _P, _DP, _P]
    lib.dsp_quantize_herm16.restype = _I
    lib.dsp_quantize_herm16.argtypes = [_P, _I, _I, _I, _P, _P, _P]
    lib.dsp_info.restype = _I
    lib.dsp_info.argtypes = [_P, ctypes.POINTER(InfoC)]
    lib.dsp_export_system.restype = _I
    lib.dsp_export_system.argtypes = [_P, _P, _P, _P]
    lib.dsp_alias_table.restype = _I
    lib.dsp_alias_table.argtypes = [_P, _IP, _IP, _IP]
    lib.dsp_geometry_counts.restype = _I
    lib.dsp_geometry_counts.argtypes = [ctypes.POINTER(ScanC), ctypes.POINTER(OpticsC), _I,
                                        ctypes.POINTER(_I), ctypes.POINTER(_I), _IP]
    lib.dsp_alias_geometry.restype = _I
    lib.dsp_alias_geometry.argtypes = [ctypes.POINTER(ScanC), ctypes.POINTER(OpticsC), _I, _IP, _IP, _IP]
    lib.dsp_active_bf.restype = _I
    lib.dsp_active_bf.argtypes = [_DP, _I, ctypes.POINTER(OpticsC), _IP, ctypes.POINTER(_I)]
    lib.dsp_band_count.restype = _I
    lib.dsp_band_count.argtypes = [ctypes.POINTER(ScanC), _DP, ctypes.POINTER(_I)]
    lib.dsp_chi_host.restype = _I
    lib.dsp_chi_host.argtypes = [ctypes.POINTER(OpticsC), _DP, _I, _DP]
    lib.dsp_chi_shift_host.restype = _I
    lib.dsp_chi_shift_host.argtypes = [ctypes.POINTER(OpticsC), _DP, _DP, _I, _DP]
    lib.dsp_sincos_host.restype = _I
    lib.dsp_sincos_host.argtypes = [_DP, _I, _DP, _DP]
    lib.dsp_atan2_host.restype = _I
    lib.dsp_atan2_host.argtypes = [_DP, _DP, _I, _DP]
    return lib
