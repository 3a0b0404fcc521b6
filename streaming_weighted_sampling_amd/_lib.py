"""ctypes declarations of libnexus.so (include/nexus.h).  Marshalling only."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnexus.so")

NX_OK = 0
NX_EINVAL = -1
NX_EALIAS = -2
NX_EWORKSPACE = -3
NX_EUNSUPPORTED = -4
NX_ENONFINITE = -5
NX_EHIP = -6
NX_COMPACT_COPY = 0
NX_COMPACT_INPLACE = 1
NX_HEADS_UNIFORM = 0
NX_HEADS_GIVEN = 1
NX_HEADS_ALLOC = 2
NX_MAX_ALLOC_HEADS = 256
NX_SCRATCH_BYTES = 16 << 20
NX_BF16 = 0
NX_F32 = 1


class NxDesc(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("lambda_", ctypes.c_float),
        ("eps_tie", ctypes.c_float),
        ("n_sink", ctypes.c_int32),
        ("n_recent", ctypes.c_int32),
        ("layer", ctypes.c_uint32),
        ("step", ctypes.c_uint32),
        ("seq_id", ctypes.c_uint32),
        ("max_out_rows", ctypes.c_int32),
        ("kv_head_stride", ctypes.c_int64),
        ("out_head_stride", ctypes.c_int64),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("n_avg", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("compact", ctypes.c_int32),
        ("head_alloc", ctypes.c_int32),
        ("head_floor", ctypes.c_int32),
        ("out_w", ctypes.c_void_p),
    ]


class NxUnit(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("keep", ctypes.c_void_p),
        ("out_k", ctypes.c_void_p),
        ("out_v", ctypes.c_void_p),
        ("app_k", ctypes.c_void_p),
        ("app_v", ctypes.c_void_p),
        ("kv_head_stride", ctypes.c_int64),
        ("out_head_stride", ctypes.c_int64),
        ("n_tokens", ctypes.c_int32),
        ("budget", ctypes.c_int32),
        ("n_append", ctypes.c_int32),
        ("layer", ctypes.c_uint32),
        ("seq_id", ctypes.c_uint32),
        ("head_cap", ctypes.c_int32),
        ("head_budget", ctypes.c_void_p),
        ("out_w", ctypes.c_void_p),
        ("head_tokens", ctypes.c_void_p),
        ("head_tokens_out", ctypes.c_void_p),
    ]


_P = ctypes.POINTER
_VP = ctypes.c_void_p
_I32 = ctypes.c_int32

SIGNATURES = {
    "nx_evict_workspace_bytes": (ctypes.c_size_t, [_P(NxDesc), _I32, _I32, _I32]),
    "nx_evict_step": (_I32, [_P(NxDesc), _VP, _VP, _VP, _I32, _I32, _I32, ctypes.c_uint64,
                             _VP, _VP, _VP]),
    "nx_evict_step_noalloc": (_I32, [_P(NxDesc), _VP, _VP, _VP, _I32, _I32, _I32, ctypes.c_uint64,
                                     _VP, _VP, _VP]),
    "nx_evict_batch": (_I32, [_P(NxDesc), _VP, _I32, _I32, _I32, ctypes.c_uint64]),
    "nx_nexus_weights": (_I32, [_P(NxDesc), _VP, _VP, _I32, _I32, _VP]),
    "nx_reservoir_select": (_I32, [_P(NxDesc), _VP, _I32, _I32, ctypes.c_uint64, _VP, _VP]),
    "nx_kv_compact": (_I32, [_P(NxDesc), _VP, _VP, _VP, _I32, _I32, _VP, _VP]),
    "nx_head_budgets": (_I32, [_P(NxDesc), _VP, _I32, _I32, _I32, _VP]),
    "nx_read_device_status": (_I32, [_P(NxDesc)]),
    "nx_stream_read": (_I32, [_VP, ctypes.c_size_t, _I32, _I32, _VP, _VP]),
    "nx_status_str": (ctypes.c_char_p, [_I32]),
    "nx_profile_enable": (_I32, [_I32]),
    "nx_profile_read": (_I32, [_P(ctypes.c_float), _P(_I32), _I32]),
    "nx_stage_name": (ctypes.c_char_p, [_I32]),
}

_lib = None


class NexusError(RuntimeError):
    def __init__(self, code, what=""):
        self.code = code
        super().__init__(f"{what}: {status_str(code)}" if what else status_str(code))


def load():
    """The loaded library; raises if libnexus.so was not built (no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m streaming_weighted_sampling_amd._build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_str(code):
    return load().nx_status_str(int(code)).decode()


def check(code, what=""):
    if code != NX_OK:
        raise NexusError(code, what)
    return code
