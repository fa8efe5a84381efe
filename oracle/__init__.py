"""Python access to the CPU oracle (``kivi_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  The product library
(``kv_cache_quantization_amd``) never imports it, and this package imports
nothing from the product library.

The arithmetic lives in plain C (``kivi_oracle.c``, built with
``-O2 -fno-fast-math -ffp-contract=off``); this module only marshals numpy
arrays.  See the C file's header for the pages and sections each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kivi_oracle.c")
_LIB = os.path.join(_HERE, "libkivi_oracle.so")

POLICY_WINDOW = 0
POLICY_PAPER = 1
POLICY_SEGMENT = 2      # KCVT: one key group per channel and flush segment

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
            "-shared", "-std=c99", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if (not os.path.exists(_LIB)
                or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_group_quant.argtypes = [P, i32, i32, P, P, P, P, P]
        L.oracle_dequant_one.restype = ctypes.c_float
        L.oracle_dequant_one.argtypes = [ctypes.c_uint8, ctypes.c_uint16, ctypes.c_uint16]
        L.oracle_quantized_prefix.argtypes = [i64, i32, i32, i32, P, P]
        L.oracle_build_cache.argtypes = [P, P, i32, i32, i32, i64, i32, i32, i32,
                                         i64, i64, P, P, P, P, P, P]
        L.oracle_dequant_cache.argtypes = [P, P, i32, i32, i32, i64, i32, i32,
                                           i64, i64, P, P, P, P, P, P, P, P]
        L.oracle_dequant_cache_kv.argtypes = [P, P, i32, i32, i32, i64, i32, i32, i32,
                                              i64, i64, P, P, P, P, P, P, P, P]
        L.oracle_build_cache_segments.argtypes = [P, P, i32, i32, i32, i64, i32, i32, P, i32,
                                                  P, P, P, P, P, P]
        L.oracle_pack_blocks_kv2.argtypes = [i32, i32, i32, i32, i64, i64, i32, i64, i64,
                                             P, P, P, P, P, P, P, P]
        L.oracle_decode_attn.argtypes = [P, P, P, i32, i32, i32, i64, i32, f64, P]
        L.oracle_attn_queries.argtypes = [P, P, P, i32, i32, i32, i64, i64, i32, f64, i32, P]
        L.oracle_block_bytes.restype = i64
        L.oracle_block_bytes.argtypes = [i32]
        L.oracle_block_bytes_g.restype = i64
        L.oracle_block_bytes_g.argtypes = [i32, i32]
        L.oracle_pack_blocks.argtypes = [i32, i32, i64, i32, i64, P, P, P, P, P, P, P]
        L.oracle_pack_blocks_kv.argtypes = [i32, i32, i32, i64, i64, i32, i64, i64,
                                            P, P, P, P, P, P, P, P]
        L.oracle_code_position.argtypes = [i32, i32, i32, i32, P, P]
        L.oracle_key_outliers.argtypes = [P, i32, i32, i32, i64, i32, i32, i64, i32,
                                          P, P, P, P, P]
        L.oracle_apply_key_outliers.argtypes = [i32, i32, i64, i32, i32, i64, i32, P, P, P]
        L.oracle_pack_outlier_records.argtypes = [i32, i32, i64, i32, i64, P, P, P]
        L.oracle_fake_quant_2d.argtypes = [P, i32, i32, i32, i32, i32, i32, P]
        L.oracle_f16_to_f32_array.argtypes = [P, P, i64]
        L.oracle_f32_to_f16_array.argtypes = [P, P, i64]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _kv(x):
    """Return (contiguous array, dtype code): 0 = fp16 bits, 1 = float32."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16), 0
    if x.dtype == np.float32:
        return x, 1
    raise TypeError("K/V must be float16 or float32, got %s" % x.dtype)


# --------------------------------------------------------------------------
# scalar building blocks
# --------------------------------------------------------------------------
def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_f16_to_f32_array(_p(h), _p(out), h.size)
    return out


def f32_to_f16(f: np.ndarray) -> np.ndarray:
    """Round float32 values to fp16 bit patterns (uint16)."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().oracle_f32_to_f16_array(_p(f), _p(out), f.size)
    return out


def group_quant(g, bits: int):
    """GroupQuant of one group: returns (codes u8, mn f32, s f32, zero16, scale16)."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    codes = np.empty(g.size, np.uint8)
    mn = np.zeros(1, np.float32)
    s = np.zeros(1, np.float32)
    z = np.zeros(1, np.uint16)
    sc = np.zeros(1, np.uint16)
    lib().oracle_group_quant(_p(g), g.size, bits, _p(codes), _p(mn), _p(s), _p(z), _p(sc))
    return codes, float(mn[0]), float(s[0]), int(z[0]), int(sc[0])


def dequant_one(code: int, zero16: int, scale16: int) -> float:
    return float(lib().oracle_dequant_one(code, zero16, scale16))


def quantized_prefix(n: int, group: int, residual: int, policy: int = POLICY_WINDOW):
    qk = ctypes.c_int64()
    qv = ctypes.c_int64()
    lib().oracle_quantized_prefix(n, group, residual, policy,
                                  ctypes.byref(qk), ctypes.byref(qv))
    return qk.value, qv.value


# --------------------------------------------------------------------------
# whole-cache views
# --------------------------------------------------------------------------
def segment_ends(appends, residual: int, deferred=()):
    """Flush segments of the segment (KCVT) policy for a sequence of appends
    of `appends[i]` tokens each: every append that moves the quantized
    prefix Q(n) = n - n mod R quantizes the tokens [Q_old, Q_new) as one
    segment.  `deferred`: indices of appends that only buffer their rows
    (the next one that does not folds them into its segment).  Returns the
    list of segment ends."""
    n, q, ends = 0, 0, []
    for i, m in enumerate(appends):
        n += m
        if i in deferred:
            continue
        qn, _ = quantized_prefix(n, 32, residual, POLICY_SEGMENT)
        if qn > q:
            ends.append(qn)
            q = qn
    return ends


def build_cache(k, v, bits: int, group: int, residual: int,
                policy: int = POLICY_WINDOW, key_outliers: int = 0, segments=None) -> dict:
    """Logical KIVI cache of K, V ([B, H, n, D], float16 or float32).
    key_outliers > 0: per key group, that many channels kept in fp16
    (oracle_key_outliers): kout_idx [B, H, qk/G, n], kout_val fp16 bits
    [B, H, qk/G, n, G].
    policy = POLICY_SEGMENT (KCVT): `segments` lists the flush segment ends
    (segment_ends); keys get one group per (segment, channel), stored per
    32-token block ("Gk" = 32), values one group per token over all D
    channels ("Gv" = D; `group` must be D)."""
    if policy == POLICY_SEGMENT:
        return _build_cache_segments(k, v, bits, group, residual, segments)
    kk, dt = _kv(k)
    vv, dt2 = _kv(v)
    assert dt == dt2 and kk.shape == vv.shape
    B, H, n, D = kk.shape
    qk, qv = quantized_prefix(n, group, residual, policy)
    c = dict(
        B=B, H=H, n=n, D=D, G=group, bits=bits, R=residual, policy=policy,
        qk=qk, qv=qv,
        kcodes=np.zeros((B, H, qk, D), np.uint8),
        kzero16=np.zeros((B, H, qk // group, D), np.uint16),
        kscale16=np.zeros((B, H, qk // group, D), np.uint16),
        vcodes=np.zeros((B, H, qv, D), np.uint8),
        vzero16=np.zeros((B, H, qv, D // group), np.uint16),
        vscale16=np.zeros((B, H, qv, D // group), np.uint16),
    )
    lib().oracle_build_cache(_p(kk), _p(vv), dt, B, H, n, D, group, bits, qk, qv,
                             _p(c["kcodes"]), _p(c["kzero16"]), _p(c["kscale16"]),
                             _p(c["vcodes"]), _p(c["vzero16"]), _p(c["vscale16"]))
    c["key_outliers"] = key_outliers
    if key_outliers > 0:
        c["kout_idx"] = np.zeros((B, H, qk // group, key_outliers), np.int32)
        c["kout_val"] = np.zeros((B, H, qk // group, key_outliers, group), np.uint16)
        lib().oracle_key_outliers(_p(kk), dt, B, H, n, D, group, qk, key_outliers,
                                  _p(c["kcodes"]), _p(c["kzero16"]), _p(c["kscale16"]),
                                  _p(c["kout_idx"]), _p(c["kout_val"]))
    # the full-precision residual, verbatim in the input dtype
    c["k_resid"] = np.ascontiguousarray(np.asarray(k)[:, :, qk:, :])
    c["v_resid"] = np.ascontiguousarray(np.asarray(v)[:, :, qv:, :])
    return c


def _build_cache_segments(k, v, bits, group, residual, segments):
    kk, dt = _kv(k)
    vv, dt2 = _kv(v)
    assert dt == dt2 and kk.shape == vv.shape
    B, H, n, D = kk.shape
    assert group == D, "KCVT values: one group over all D channels"
    ends = np.ascontiguousarray(np.asarray(list(segments or []), dtype=np.int64))
    assert all(int(e) % 32 == 0 for e in ends) and list(ends) == sorted(set(ends.tolist()))
    Q = int(ends[-1]) if len(ends) else 0
    assert Q <= n
    c = dict(
        B=B, H=H, n=n, D=D, G=group, Gk=32, Gv=D, bits=bits, R=residual,
        policy=POLICY_SEGMENT, qk=Q, qv=Q, segments=[int(e) for e in ends],
        kcodes=np.zeros((B, H, Q, D), np.uint8),
        kzero16=np.zeros((B, H, Q // 32, D), np.uint16),
        kscale16=np.zeros((B, H, Q // 32, D), np.uint16),
        vcodes=np.zeros((B, H, Q, D), np.uint8),
        vzero16=np.zeros((B, H, Q, 1), np.uint16),
        vscale16=np.zeros((B, H, Q, 1), np.uint16),
        key_outliers=0,
    )
    lib().oracle_build_cache_segments(_p(kk), _p(vv), dt, B, H, n, D, bits, _p(ends), len(ends),
                                      _p(c["kcodes"]), _p(c["kzero16"]), _p(c["kscale16"]),
                                      _p(c["vcodes"]), _p(c["vzero16"]), _p(c["vscale16"]))
    c["k_resid"] = np.ascontiguousarray(np.asarray(k)[:, :, Q:, :])
    c["v_resid"] = np.ascontiguousarray(np.asarray(v)[:, :, Q:, :])
    return c


def dequant_cache(k, v, cache: dict):
    """Float32 K_hat, V_hat [B, H, n, D] of the cache built from k, v."""
    kk, dt = _kv(k)
    vv, _ = _kv(v)
    B, H, n, D = kk.shape
    khat = np.empty((B, H, n, D), np.float32)
    vhat = np.empty((B, H, n, D), np.float32)
    lib().oracle_dequant_cache_kv(
        _p(kk), _p(vv), dt, B, H, n, D, cache.get("Gk", cache["G"]), cache.get("Gv", cache["G"]),
        cache["qk"], cache["qv"],
        _p(cache["kcodes"]), _p(cache["kzero16"]), _p(cache["kscale16"]),
        _p(cache["vcodes"]), _p(cache["vzero16"]), _p(cache["vscale16"]),
        _p(khat), _p(vhat))
    if cache.get("key_outliers", 0) > 0:
        lib().oracle_apply_key_outliers(B, H, n, D, cache["G"], cache["qk"], cache["key_outliers"],
                                        _p(cache["kout_idx"]), _p(cache["kout_val"]), _p(khat))
    return khat, vhat


def decode_attn(q, khat, vhat, sm_scale: float | None = None) -> np.ndarray:
    """softmax(q K_hat^T * sm_scale) V_hat per query head, fp64 accumulation.

    q: [B, Hq, D] (any float dtype, converted to float32); khat, vhat:
    [B, H, n, D] float32.  Query head hq reads KV head hq // (Hq // H)."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float32))
    khat = np.ascontiguousarray(khat, dtype=np.float32)
    vhat = np.ascontiguousarray(vhat, dtype=np.float32)
    B, Hq, D = q.shape
    _, H, n, _ = khat.shape
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, D), np.float32)
    lib().oracle_decode_attn(_p(q), _p(khat), _p(vhat), B, H, Hq, n, D,
                             float(sm_scale), _p(out))
    return out


def attn_queries(q, khat, vhat, causal: bool = False, sm_scale: float | None = None) -> np.ndarray:
    """T queries per query head: softmax(q K_hat^T * sm_scale [+ mask]) V_hat,
    fp64 accumulation.  q: [B, Hq, T, D]; khat, vhat: [B, H, n, D] float32.
    causal: query t is token n - T + t and sees tokens 0 .. n - T + t."""
    q = np.ascontiguousarray(np.asarray(q, dtype=np.float32))
    khat = np.ascontiguousarray(khat, dtype=np.float32)
    vhat = np.ascontiguousarray(vhat, dtype=np.float32)
    B, Hq, T, D = q.shape
    _, H, n, _ = khat.shape
    if causal and T > n:
        raise ValueError("causal attention needs T <= n")
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(D)
    out = np.empty((B, Hq, T, D), np.float32)
    lib().oracle_attn_queries(_p(q), _p(khat), _p(vhat), B, H, Hq, T, n, D, float(sm_scale),
                              int(bool(causal)), _p(out))
    return out


def block_bytes(bits: int, Gv: int = 32) -> int:
    """Bytes of one 32-token block when value groups span Gv channels (the
    split layout when Gv > 32; see oracle_block_bytes_g)."""
    return int(lib().oracle_block_bytes_g(bits, Gv))


def is_split(cache: dict) -> bool:
    """The split layout (key zero / scale once per key group in a separate
    array) is used when value groups span more than 32 channels."""
    return cache.get("Gv", cache["G"]) > 32


def kunit_tokens(cache: dict) -> int:
    """Tokens per key unit of the split layout: the key group size."""
    return cache.get("Gk", cache["G"])


def pack_cache(cache: dict, max_groups: int | None = None, max_kunits: int | None = None):
    """(blocks, kside): the packed 32-token blocks [B*H, max_groups,
    block_bytes] (u8) of the quantized tokens -- keys of the first qk,
    values of the first qv (a value row at or past qv inside a block that
    holds value rows packs as 0) -- and, in the split layout, the key units
    [B*H, max_kunits, 2, D] (fp16 bits: K scale, K zero of each key group),
    else None.  See oracle_pack_blocks_kv2 for the two layouts."""
    assert cache["D"] == 128 and cache["G"] in (32, 64, 128)
    B, H, qk, qv, bits = cache["B"], cache["H"], cache["qk"], cache["qv"], cache["bits"]
    Gk, Gv = kunit_tokens(cache), cache.get("Gv", cache["G"])
    ng = max(qk // 32, -(-qv // 32))
    if max_groups is None:
        max_groups = ng
    assert max_groups >= ng
    out = np.zeros((B * H, max_groups, block_bytes(bits, Gv)), np.uint8)
    kside = None
    if is_split(cache):
        if max_kunits is None:
            max_kunits = qk // Gk
        assert max_kunits >= qk // Gk
        kside = np.zeros((B * H, max_kunits, 2, 128), np.uint16)
    lib().oracle_pack_blocks_kv2(B, H, Gk, Gv, qk, qv, bits, max_groups,
                                 max_kunits or 0,
                                 _p(cache["kcodes"]), _p(cache["kzero16"]), _p(cache["kscale16"]),
                                 _p(cache["vcodes"]), _p(cache["vzero16"]), _p(cache["vscale16"]),
                                 _p(out), _p(kside) if kside is not None else None)
    return out, kside


def pack_blocks(cache: dict, max_groups: int | None = None) -> np.ndarray:
    """The packed blocks of pack_cache (without the key units)."""
    return pack_cache(cache, max_groups)[0]


def pack_outlier_records(cache: dict, max_groups: int | None = None) -> np.ndarray:
    """Outlier records [B*H, max_groups, 256] (u8) of a cache built with
    key_outliers > 0 at G = 32 (see oracle_pack_outlier_records)."""
    assert cache["G"] == 32 and cache["key_outliers"] > 0
    B, H, qk = cache["B"], cache["H"], cache["qk"]
    if max_groups is None:
        max_groups = qk // 32
    out = np.zeros((B * H, max_groups, 256), np.uint8)
    lib().oracle_pack_outlier_records(B, H, qk, cache["key_outliers"], max_groups,
                                      _p(cache["kout_idx"]), _p(cache["kout_val"]), _p(out))
    return out


def code_position(bits: int, is_v: bool, token: int, channel: int):
    d = ctypes.c_int64()
    b = ctypes.c_int()
    lib().oracle_code_position(bits, int(is_v), token, channel,
                               ctypes.byref(d), ctypes.byref(b))
    return d.value, b.value


def fake_quant_2d(x, axis: int, bits: int, group: int, mode: int = 0) -> np.ndarray:
    """Notebook-style reconstruction of a 2-D float32 array (see the C file)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    assert (rows if axis == 0 else cols) % group == 0
    out = np.empty_like(x)
    lib().oracle_fake_quant_2d(_p(x), rows, cols, axis, bits, group, mode, _p(out))
    return out
