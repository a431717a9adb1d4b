"""ctypes view of librpa_probes.so (include/rpa_probes.h): measurement probes
of the GPU (HBM streaming, dense bf16 MFMA with its shader clock, VALU issue
rates, LDS and global -> LDS rates) that the benchmark reports as measured
ceilings beside the published peaks.  Only argument marshalling lives here; the attention path never uses
this library."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librpa_probes.so")
EXPORTS = ("rpa_probe_read", "rpa_probe_copy", "rpa_probe_mfma", "rpa_probe_valu",
           "rpa_probe_lds", "rpa_probe_dma", "rpa_probe_lds_dma", "rpa_probe_mix",
           "rpa_probe_lds_mfma", "rpa_probe_mix_vgpr_acc")
VALU_OPS = {"exp": 0, "rcp": 1, "fma": 2}
# LDS op -> bytes per instruction and wave
LDS_OPS = {"ds_read_b128": (0, 1024), "ds_read_b64_tr_b16": (1, 512), "ds_write_b128": (2, 1024)}
# LDS-fed MFMA patterns
LDS_MFMA_MODES = {"qk_lds_2acc": 0, "pv_lds_4acc": 1, "qk_regs_2acc": 2, "qk_lds_4acc": 3}

_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m ragged_paged_kv_scatter_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.rpa_probe_read.argtypes = [P, SZ, P, I, P]
    lib.rpa_probe_copy.argtypes = [P, P, SZ, I, P]
    lib.rpa_probe_mfma.argtypes = [P, P, I, I, P]
    lib.rpa_probe_valu.argtypes = [P, I, I, I, P]
    lib.rpa_probe_lds.argtypes = [P, P, I, I, I, P]
    lib.rpa_probe_dma.argtypes = [P, SZ, P, P, I, I, P]
    lib.rpa_probe_lds_dma.argtypes = [P, SZ, P, P, I, ctypes.c_int64, I, P]
    lib.rpa_probe_mix.argtypes = [P, P, I, I, I, I, P]
    lib.rpa_probe_mix_vgpr_acc.argtypes = [P, P, I, I, I, I, P]
    lib.rpa_probe_lds_mfma.argtypes = [P, P, I, I, I, P]
    for n in EXPORTS:
        getattr(lib, n).restype = ctypes.c_int
    _lib = lib
    return lib


def check(code, what):
    if code != 0:
        raise RuntimeError(f"{what} failed with HIP error {code}")
