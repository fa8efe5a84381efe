"""ctypes binding of libkivi (include/kivi.h).

Argument marshalling only: every step of quantization, flush and decode
attention runs in the HIP kernels of ``libkivi.so``.  PyTorch provides device
memory and the current HIP stream, nothing else.  There is no fallback: if
the library is not built, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KIVI_LIB") or os.path.join(HERE, "libkivi.so")

KIVI_OK = 0
KIVI_ERR_INVALID_ARG = 1
KIVI_ERR_UNSUPPORTED = 2
KIVI_ERR_CAPACITY = 3
KIVI_ERR_BUFFER_TOO_SMALL = 4
KIVI_ERR_STATE = 5
KIVI_ERR_HIP = 6

KIVI_F16 = 0
KIVI_F32 = 1
KIVI_FLUSH_WINDOW = 0
KIVI_FLUSH_PAPER = 1
KIVI_FLUSH_SEGMENT = 2      # KCVT: one key group per channel and flush segment
KIVI_DEFER_FLUSH = 1
KIVI_NOALLOC_SCRATCH_BYTES = 32 << 20      # fixed decode scratch of kivi_decode_attn_noalloc

# Every symbol include/kivi.h declares.
EXPORTED = (
    "kivi_cache_bytes", "kivi_cache_create", "kivi_cache_destroy", "kivi_append",
    "kivi_flush", "kivi_plan_append", "kivi_decode_workspace_bytes",
    "kivi_decode_plan", "kivi_decode_attn", "kivi_decode_attn_noalloc", "kivi_append_decode",
    "kivi_attn",
    "kivi_attn_workspace_bytes",
    "kivi_attn_plan", "kivi_get_layout", "kivi_status_string",
)


class kivi_config(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
        ("residual", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("policy", ctypes.c_int32), ("key_outliers", ctypes.c_int32),
        ("max_tokens", ctypes.c_int64),
    ]


class kivi_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "blocks", "ring_k", "ring_v", "block_bytes", "code_bytes", "off_kcode",
        "off_vcode", "off_kscale", "off_kzero", "off_vscale", "off_vzero")] + [
        ("max_groups", ctypes.c_int64), ("ring_capacity", ctypes.c_int64),
        ("n_tokens", ctypes.c_int64), ("n_quantized", ctypes.c_int64),
        ("n_vquantized", ctypes.c_int64), ("outliers", ctypes.c_size_t),
        ("kside", ctypes.c_size_t), ("kside_unit_tokens", ctypes.c_int64),
        ("max_kside_units", ctypes.c_int64)]


class kivi_append_plan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "n_old", "n_new_total", "q_old", "q_new", "flush_token_begin",
        "flush_token_end", "ring_token_begin", "ring_token_end",
        "v_flush_token_begin", "v_flush_token_end")]


class KiviError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (where, kivi_status_string(status), status))


_lib = None


def lib():
    """Load libkivi.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkivi.so is not built (%s); run "
                               "`python -m kv_cache_quantization_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz, u32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_size_t, ctypes.c_uint32)
        L.kivi_cache_bytes.restype = sz
        L.kivi_cache_bytes.argtypes = [ctypes.POINTER(kivi_config)]
        L.kivi_cache_create.restype = i32
        L.kivi_cache_create.argtypes = [ctypes.POINTER(kivi_config), P, sz, ctypes.POINTER(P)]
        L.kivi_cache_destroy.restype = i32
        L.kivi_cache_destroy.argtypes = [P]
        L.kivi_append.restype = i32
        L.kivi_append.argtypes = [P, P, P, i64, u32, P]
        L.kivi_flush.restype = i32
        L.kivi_flush.argtypes = [P, P]
        L.kivi_plan_append.restype = i32
        L.kivi_plan_append.argtypes = [P, i64, ctypes.POINTER(kivi_append_plan)]
        L.kivi_decode_workspace_bytes.restype = sz
        L.kivi_decode_workspace_bytes.argtypes = [P]
        L.kivi_decode_plan.restype = i32
        L.kivi_decode_plan.argtypes = [P, ctypes.POINTER(i32), ctypes.POINTER(i32)]
        L.kivi_decode_attn.restype = i32
        L.kivi_decode_attn.argtypes = [P, P, i32, ctypes.c_float, P, P, sz, P]
        L.kivi_decode_attn_noalloc.restype = i32
        L.kivi_decode_attn_noalloc.argtypes = [P, P, i32, ctypes.c_float, P, P]
        L.kivi_append_decode.restype = i32
        L.kivi_append_decode.argtypes = [P, P, P, i64, P, i32, ctypes.c_float, P, P, sz, P]
        L.kivi_attn.restype = i32
        L.kivi_attn.argtypes = [P, P, i32, i64, i32, ctypes.c_float, P, P, sz, P]
        L.kivi_attn_workspace_bytes.restype = sz
        L.kivi_attn_workspace_bytes.argtypes = [P, i64]
        L.kivi_attn_plan.restype = i32
        L.kivi_attn_plan.argtypes = [P, i64, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                     ctypes.POINTER(i32)]
        L.kivi_get_layout.restype = i32
        L.kivi_get_layout.argtypes = [P, ctypes.POINTER(kivi_layout)]
        L.kivi_status_string.restype = ctypes.c_char_p
        L.kivi_status_string.argtypes = [i32]
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != KIVI_OK:
        raise KiviError(status, where)


# ---------------------------------------------------------------------------
# One Python function per C entry point, same names.
# ---------------------------------------------------------------------------
def kivi_status_string(status: int) -> str:
    return lib().kivi_status_string(status).decode()


def kivi_cache_bytes(cfg: kivi_config) -> int:
    return int(lib().kivi_cache_bytes(ctypes.byref(cfg)))


def kivi_cache_create(cfg: kivi_config, dev_mem: int, dev_bytes: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().kivi_cache_create(ctypes.byref(cfg), dev_mem, dev_bytes, ctypes.byref(h)),
           "kivi_cache_create")
    return h.value


def kivi_cache_destroy(handle: int) -> None:
    _check(lib().kivi_cache_destroy(handle), "kivi_cache_destroy")


def kivi_append(handle: int, k: int, v: int, n_new: int, flags: int, stream: int) -> None:
    _check(lib().kivi_append(handle, k, v, n_new, flags, stream), "kivi_append")


def kivi_flush(handle: int, stream: int) -> None:
    _check(lib().kivi_flush(handle, stream), "kivi_flush")


def kivi_plan_append(handle: int, n_new: int) -> kivi_append_plan:
    p = kivi_append_plan()
    _check(lib().kivi_plan_append(handle, n_new, ctypes.byref(p)), "kivi_plan_append")
    return p


def kivi_decode_workspace_bytes(handle: int) -> int:
    return int(lib().kivi_decode_workspace_bytes(handle))


def kivi_decode_plan(handle: int):
    s, g = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().kivi_decode_plan(handle, ctypes.byref(s), ctypes.byref(g)), "kivi_decode_plan")
    return s.value, g.value


def kivi_decode_attn(handle: int, q: int, q_dtype: int, softmax_scale: float, out: int,
                     workspace: int, ws_bytes: int, stream: int) -> None:
    _check(lib().kivi_decode_attn(handle, q, q_dtype, softmax_scale, out, workspace,
                                  ws_bytes, stream), "kivi_decode_attn")


def kivi_decode_attn_noalloc(handle: int, q: int, q_dtype: int, softmax_scale: float, out: int,
                             stream: int) -> None:
    _check(lib().kivi_decode_attn_noalloc(handle, q, q_dtype, softmax_scale, out, stream),
           "kivi_decode_attn_noalloc")


def kivi_append_decode(handle: int, k: int, v: int, n_new: int, q: int, q_dtype: int,
                       softmax_scale: float, out: int, workspace: int, ws_bytes: int,
                       stream: int) -> None:
    _check(lib().kivi_append_decode(handle, k, v, n_new, q, q_dtype, softmax_scale, out,
                                    workspace, ws_bytes, stream), "kivi_append_decode")


def kivi_attn(handle: int, q: int, q_dtype: int, T: int, causal: int, softmax_scale: float,
              out: int, workspace: int, ws_bytes: int, stream: int) -> None:
    _check(lib().kivi_attn(handle, q, q_dtype, T, causal, softmax_scale, out, workspace,
                           ws_bytes, stream), "kivi_attn")


def kivi_attn_workspace_bytes(handle: int, T: int) -> int:
    return int(lib().kivi_attn_workspace_bytes(handle, T))


def kivi_attn_plan(handle: int, T: int):
    qb, s, g = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().kivi_attn_plan(handle, T, ctypes.byref(qb), ctypes.byref(s), ctypes.byref(g)),
           "kivi_attn_plan")
    return qb.value, s.value, g.value


def kivi_get_layout(handle: int) -> kivi_layout:
    lo = kivi_layout()
    _check(lib().kivi_get_layout(handle, ctypes.byref(lo)), "kivi_get_layout")
    return lo


def make_config(batch, n_kv_heads, n_q_heads, head_dim=128, bits=2, group=32, residual=128,
                max_tokens=4096, kv_dtype=KIVI_F16, policy=KIVI_FLUSH_WINDOW,
                key_outliers=0) -> kivi_config:
    return kivi_config(batch, n_kv_heads, n_q_heads, head_dim, bits, group, residual,
                       kv_dtype, policy, key_outliers, max_tokens)
