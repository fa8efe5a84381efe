"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no KIVI arithmetic: it only draws random K, V and q with
the shapes and value distributions of the workloads the pages describe.

* The notebook workload ("KIVI - 2-bit KV cache quantisation", section "K
  (per-channel) and V (per-token) quantisation"): T = 1024 tokens, head_dim
  128, float32 K and V ~ N(0, 0.5^2) drawn with torch's CPU generator from
  seed 0 (K first, then V), channels 3, 17, 40, 88 of K scaled by 5; the
  query is row 0 of the notebook's Q (seed 1, shape [1, 1024, 128]).
* The serving workloads (Llama-3-8B-like layers: 8 KV heads, 32 query heads,
  head_dim 128): K and V ~ N(0, 1) in float32, 4 outlier channels per KV head
  (the same for every batch entry) scaled by 5 on K only, then rounded to
  float16; queries ~ N(0, 1) in float16.  Keys carry channel outliers and
  values do not, as in the paper review's analysis of key/value
  distributions ("[Paper review] KIVI ...", 3.1.2).

Two generators draw the serving workloads: ``*_host`` (numpy PCG64, one
independent stream per (tensor, batch, head, chunk), so any stream can be
regenerated alone) for sizes the CPU oracle handles, and ``*_device`` (a
torch generator on the GPU) for the multi-gigabyte configurations, whose
sampled streams are copied back to the host when checked.
"""
from __future__ import annotations

import hashlib

import numpy as np

OUTLIER_SCALE = 5.0
N_OUTLIERS = 4
TENSOR_K, TENSOR_V, TENSOR_Q = 0, 1, 2


def notebook_inputs():
    """(K, V, q) of the notebook workload as float32 numpy arrays
    K, V: [1, 1, 1024, 128]; q: [1, 1, 128]."""
    import torch
    g = torch.Generator().manual_seed(0)
    T, D = 1024, 128
    K = torch.randn(T, D, generator=g) * 0.5
    V = torch.randn(T, D, generator=g) * 0.5
    for c in (3, 17, 40, 88):
        K[:, c] *= OUTLIER_SCALE
    gq = torch.Generator().manual_seed(1)
    Q = torch.randn(1, T, D, generator=gq)
    return (K.numpy().reshape(1, 1, T, D).copy(), V.numpy().reshape(1, 1, T, D).copy(),
            Q[0, :1].numpy().reshape(1, 1, D).copy())


def outlier_channels(cfg_id: int, n_kv_heads: int, head_dim: int = 128) -> np.ndarray:
    """[H, 4] distinct outlier channels per KV head."""
    out = np.empty((n_kv_heads, N_OUTLIERS), np.int64)
    for h in range(n_kv_heads):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, 9, h])))
        out[h] = np.sort(rng.choice(head_dim, N_OUTLIERS, replace=False))
    return out


def kv_host(cfg_id: int, B: int, H: int, n: int, D: int = 128, chunk: int = 0,
            dtype=np.float16):
    """(K, V) [B, H, n, D] drawn per stream with numpy PCG64."""
    out = []
    oc = outlier_channels(cfg_id, H, D)
    for tensor in (TENSOR_K, TENSOR_V):
        x = np.empty((B, H, n, D), np.float32)
        for b in range(B):
            for h in range(H):
                rng = np.random.Generator(np.random.PCG64(
                    np.random.SeedSequence([cfg_id, tensor, b, h, chunk])))
                x[b, h] = rng.standard_normal((n, D), dtype=np.float32)
                if tensor == TENSOR_K:
                    x[b, h][:, oc[h]] *= np.float32(OUTLIER_SCALE)
        out.append(x.astype(dtype))
    return out[0], out[1]


def queries_host(cfg_id: int, B: int, Hq: int, D: int = 128, step: int = 0,
                 dtype=np.float16):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, TENSOR_Q, step])))
    return rng.standard_normal((B, Hq, D), dtype=np.float32).astype(dtype)


def queries_multi_host(cfg_id: int, B: int, Hq: int, T: int, D: int = 128, dtype=np.float16):
    """T query rows per (batch, query head): [B, Hq, T, D], row t drawn as
    queries_host(..., step=t)."""
    return np.stack([queries_host(cfg_id, B, Hq, D, step=t, dtype=dtype) for t in range(T)],
                    axis=2)


def queries_multi_device(cfg_id: int, B: int, Hq: int, T: int, D: int = 128, device="cuda"):
    """[B, Hq, T, D] float16 query rows drawn on the device."""
    import torch
    g = torch.Generator(device=device).manual_seed(_torch_seed(cfg_id, TENSOR_Q, "multi", T))
    return torch.randn((B, Hq, T, D), generator=g, device=device,
                       dtype=torch.float32).to(torch.float16)


def _torch_seed(*key) -> int:
    h = hashlib.sha256(("kivi-synth-" + "-".join(str(k) for k in key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def kv_device(cfg_id: int, B: int, H: int, n: int, D: int = 128, chunk: int = 0,
              device="cuda", dtype=None):
    """(K, V) [B, H, n, D] float16 drawn on the device with a seeded torch generator."""
    import torch
    dtype = dtype or torch.float16
    oc = torch.as_tensor(outlier_channels(cfg_id, H, D), device=device)
    res = []
    for tensor in (TENSOR_K, TENSOR_V):
        g = torch.Generator(device=device).manual_seed(_torch_seed(cfg_id, tensor, chunk))
        x = torch.randn((B, H, n, D), generator=g, device=device, dtype=torch.float32)
        if tensor == TENSOR_K:
            scale = torch.ones((H, D), device=device)
            scale.scatter_(1, oc, OUTLIER_SCALE)
            x.mul_(scale.view(1, H, 1, D))
        res.append(x.to(dtype))
        del x
    return res[0], res[1]


def queries_device(cfg_id: int, B: int, Hq: int, D: int = 128, step: int = 0, device="cuda"):
    import torch
    g = torch.Generator(device=device).manual_seed(_torch_seed(cfg_id, TENSOR_Q, step))
    return torch.randn((B, Hq, D), generator=g, device=device).to(torch.float16)


# The five workloads (sizes only; which generator draws them is the caller's
# choice as described above).
CONFIGS = {
    1: dict(name="notebook-T1024-fp32", B=1, H=1, Hq=1, n=1024, R=0, bits=(2, 4),
            dtype="f32"),
    2: dict(name="llama3-8b-layer-n4096", B=1, H=8, Hq=32, n=4096, R=32, bits=(2,),
            dtype="f16"),
    3: dict(name="long-context-B16-n32768", B=16, H=8, Hq=32, n=32768, R=128, bits=(2,),
            dtype="f16"),
    4: dict(name="streaming-B8-prefill8192-512steps", B=8, H=8, Hq=32, n=8192 + 512,
            prefill=8192, steps=512, R=128, bits=(2,), dtype="f16"),
    5: dict(name="capacity-B32-n131072-chunk8192", B=32, H=8, Hq=32, n=131072, chunk=8192,
            R=128, bits=(2, 4), dtype="f16"),
}
