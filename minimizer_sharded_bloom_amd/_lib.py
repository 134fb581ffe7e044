"""ctypes declarations of libsbf.so (include/sbf.h).  Argument marshalling
only: every step of insert, query and probe runs in the library's kernels."""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsbf.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "sbf.h")

SBF_OK = 0
SBF_EINVAL = -1
SBF_EUNSUPPORTED = -2
SBF_ENOMEM = -3
SBF_EDEVICE = -4
SBF_EIO = -5
SBF_KIND_SBF = 0
SBF_KIND_BBF = 1
SBF_KIND_WIDE = 2
SBF_ALPHABET_DNA = 0
SBF_ALPHABET_PROTEIN = 1
SBF_ALPHABET_TRIPLET = 2
SBF_HOST = 1
SBF_DEVICE = 2


class SbfInfo(ctypes.Structure):
    _fields_ = [("k", ctypes.c_uint32), ("m", ctypes.c_uint32), ("s", ctypes.c_uint32),
                ("H", ctypes.c_uint32), ("kind", ctypes.c_uint32), ("specialized", ctypes.c_uint32),
                ("num_shards", ctypes.c_uint64), ("filter_bytes", ctypes.c_uint64),
                ("words_per_shard", ctypes.c_uint32), ("alphabet", ctypes.c_uint32)]


class SbfFastxStats(ctypes.Structure):
    _fields_ = [("records", ctypes.c_uint64), ("bases", ctypes.c_uint64), ("chunks", ctypes.c_uint64),
                ("parse_seconds", ctypes.c_double), ("total_seconds", ctypes.c_double)]


_u32, _u64, _p, _int = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int

SIGNATURES = {
    "sbf_create": (_int, [ctypes.POINTER(_p), _u32, _u32, _u32, _u32, _u64]),
    "sbf_create_bbf": (_int, [ctypes.POINTER(_p), _u32, _u32, _u64]),
    "sbf_create_wide": (_int, [ctypes.POINTER(_p), _u32, _u32, _u32, _u32, _u64]),
    "sbf_create_alphabet": (_int, [ctypes.POINTER(_p), _u32, _u32, _u32, _u32, _u32, _u64]),
    "sbf_destroy": (_int, [_p]),
    "sbf_clear": (_int, [_p, _p]),
    "sbf_info": (_int, [_p, ctypes.POINTER(SbfInfo)]),
    "sbf_copy_filter": (_int, [_p, _p, _u64, _u32, _p]),
    "sbf_filter_device_ptr": (_p, [_p]),
    "sbf_packed_words": (None, [_u64, ctypes.POINTER(_u64), ctypes.POINTER(_u64)]),
    "sbf_pack": (_int, [_p, _u64, _p, _p, _p]),
    "sbf_insert_packed": (_int, [_p, _p, _p, _u64, _p]),
    "sbf_query_packed": (_int, [_p, _p, _p, _u64, _p, _p]),
    "sbf_insert_seq": (_int, [_p, _p, _u64, _u32, _p]),
    "sbf_insert_seq_noalloc": (_int, [_p, _p, _u64, _p]),
    "sbf_query_seq": (_int, [_p, _p, _u64, _p, _u32, _p]),
    "sbf_query_reads": (_int, [_p, _p, _u64, _u32, _u64, _p, _p]),
    "sbf_fpr_probe": (_int, [_p, _u64, _u64, ctypes.POINTER(_u64)]),
    "sbf_fpr_probe_device": (_int, [_p, _u64, _u64, _p, _p]),
    "sbf_set_staging": (_int, [_p, _u64]),
    "sbf_fastx_open": (_int, [ctypes.POINTER(_p), ctypes.c_char_p]),
    "sbf_fastx_read": (_int, [_p, _p, _u64, ctypes.POINTER(_u64), _p, _u64, ctypes.POINTER(_u64)]),
    "sbf_fastx_records": (_u64, [_p]),
    "sbf_fastx_close": (_int, [_p]),
    "sbf_insert_fastx": (_int, [_p, ctypes.c_char_p, ctypes.POINTER(SbfFastxStats)]),
    "sbf_query_fastx": (_int, [_p, ctypes.c_char_p, _p, _p, _u64, ctypes.POINTER(SbfFastxStats)]),
    "sbf_membench_shard_reads": (_int, [_p, _u64, _u64, _u64, _p, _p]),
    "sbf_membench_shard_ors": (_int, [_p, _u64, _u64, _u64, _p]),
    "sbf_membench_shard_rmw": (_int, [_p, _u64, _u64, _u64, _u32, _p]),
    "sbf_membench_valu": (_int, [_u32, _u64, _p, _p]),
    "sbf_strerror": (ctypes.c_char_p, [_int]),
    "sbf_last_error": (ctypes.c_char_p, []),
}


def header_symbols(path: str = HEADER) -> list[str]:
    """Names of the functions include/sbf.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sbf_[a-z_0-9]+)\s*\(", text)))


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsbf.so; raises if it has not been built (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libsbf.so is not built (%s); run `python -m minimizer_sharded_bloom_amd.build`" % path)
    # One HIP runtime per process: torch ships its own libamdhip64.so.7 with
    # the same soname as the system one libsbf.so is linked against.  Whichever
    # is loaded first serves both, and torch cannot initialise its devices on
    # the system build.  Loading torch first binds libsbf.so to torch's
    # runtime, so device pointers and streams are shared by one runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class SbfError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s (%d): %s" % (what, code, last_error()))


def last_error() -> str:
    return (load().sbf_last_error() or b"").decode()


def check(code: int, what: str) -> None:
    if code != SBF_OK:
        raise SbfError(code, what)
