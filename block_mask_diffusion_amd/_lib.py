"""ctypes loader for libtt.so (the C ABI declared in include/tt.h).

torch is imported before the library is opened: torch ships its own HIP runtime
(SONAME libamdhip64.so.7) and libtt.so's dependency on that SONAME must resolve to the
copy torch already loaded, so device pointers and streams from torch are valid in the
library. After loading, the process maps are checked for a second HIP runtime, and the
load fails loudly if one is found. There is no fallback: without the library the
package raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the library: shares torch's HIP runtime)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtt.so")

TT_F32, TT_BF16 = 0, 1
TT_OK, TT_ERR_ARG, TT_ERR_UNSUPPORTED, TT_ERR_WORKSPACE, TT_ERR_HIP = 0, -1, -2, -3, -4

# every symbol include/tt.h declares
EXPORTS = ("tt_block_attn", "tt_context_extend", "tt_lmhead_logits", "tt_confidence_unmask",
           "tt_confidence_unmask_noalloc", "tt_unmask_sample", "tt_lmhead_unmask", "tt_status_string",
           "tt_abi_version")

TT_SAMPLER_CONFIDENCE, TT_SAMPLER_PREDICT_NOISE = 0, 1
SAMPLER_KINDS = {"confidence": TT_SAMPLER_CONFIDENCE, "predict_noise": TT_SAMPLER_PREDICT_NOISE}


class Sampler(ctypes.Structure):
    """struct tt_sampler of include/tt.h."""
    _fields_ = [("kind", ctypes.c_int), ("gamma", ctypes.c_float), ("temperature", ctypes.c_float)]

_lib = None


class TTError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def _hip_runtimes_mapped():
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_mask_diffusion_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped in this process: {sorted(runtimes)}")
    vp, i, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.POINTER(ctypes.c_size_t)
    lib.tt_block_attn.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i64, i, f32, i, vp, sz, vp]
    lib.tt_block_attn.restype = i
    lib.tt_context_extend.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i64, i, f32, i, vp, sz, vp]
    lib.tt_context_extend.restype = i
    lib.tt_lmhead_logits.argtypes = [vp, vp, vp, i, i, i, i, vp]
    lib.tt_lmhead_logits.restype = i
    lib.tt_confidence_unmask.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f32, i, vp, sz, vp]
    lib.tt_confidence_unmask.restype = i
    lib.tt_confidence_unmask_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f32, i, vp]
    lib.tt_confidence_unmask_noalloc.restype = i
    smp = ctypes.POINTER(Sampler)
    lib.tt_unmask_sample.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, smp, i, vp, sz, vp]
    lib.tt_unmask_sample.restype = i
    lib.tt_lmhead_unmask.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, smp, i, i, vp, sz, vp]
    lib.tt_lmhead_unmask.restype = i
    lib.tt_status_string.argtypes = [i]
    lib.tt_status_string.restype = ctypes.c_char_p
    lib.tt_abi_version.argtypes = []
    lib.tt_abi_version.restype = i
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().tt_status_string(int(status)).decode()
