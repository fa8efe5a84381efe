"""GPU parity of the attention of T queries per head (kivi_attn, through the
C ABI) against the oracle's attention over the same dequantized cache.

Bar: max over (b, hq, t) of |o - r|_inf / |r|_inf <= 2e-3, the decode step's
tolerance.  Cases cover both masks (none, and causal with the queries as the
last T cached tokens), 1, 2 and 4 query heads per KV head, 2, 4 and 8 bits,
query counts that leave padding columns, queries straddling the quantized
prefix and the fp16 residual, split ranges merged by the combine kernel and
a single range writing the output directly, fp32 queries, fp32 caches with
residual tokens, and the notebook's attention over all 1024 rows of its Q on
its fp32 cache.
"""
import numpy as np
import pytest

from gpu_helpers import TOL, log, new_cache, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_quantization_amd import kivi
    kivi.lib()   # fail loudly if the HIP library is missing


def _run(orc, B, H, Hq, n, T, bits, R, causal, seed, chunks=None, q_dtype=np.float16,
         label="", G=32, dtype=np.float16, policy=0):
    from kv_cache_quantization_amd import synth, kivi
    k, v = synth.kv_host(seed, B, H, n, dtype=dtype)
    q = synth.queries_multi_host(seed, B, Hq, T, dtype=q_dtype)
    cache = new_cache(B, H, Hq, max_tokens=n + 64, bits=bits, R=R, group=G, dtype=dtype,
                      policy=policy)
    pos = 0
    for c in (chunks or [n]):
        cache.append(to_dev(k[:, :, pos:pos + c]), to_dev(v[:, :, pos:pos + c]))
        pos += c
    plan = kivi.kivi_attn_plan(cache.handle, T)
    log("case %s: B=%d H=%d Hq=%d n=%d T=%d bits=%d R=%d causal=%d plan(qblocks, splits, "
        "gps)=%s" % (label, B, H, Hq, n, T, bits, R, causal, plan))
    out = cache.attn(to_dev(q), causal=causal).cpu().numpy()
    ref_cache = orc.build_cache(k, v, bits, G, R, policy)
    kh, vh = orc.dequant_cache(k, v, ref_cache)
    ref = orc.attn_queries(q, kh, vh, causal)
    e = rel_err(out, ref)
    log("  attn rel err %.3g" % e)
    assert np.isfinite(out).all(), label
    assert e <= TOL, (label, e)
    return cache, q, out


@pytest.mark.parametrize("n,T,bits,R,gq,causal", [
    (4096, 16, 2, 32, 4, 0),     # a few queries, long context: split ranges + combine
    (1000, 300, 2, 128, 4, 1),   # causal mask inside quantized groups and the residual
    (1000, 64, 4, 128, 4, 1),    # queries inside the residual only
    (777, 33, 2, 64, 2, 0),      # padding columns (33 is not a multiple of 8)
    (513, 5, 4, 0, 1, 1),        # R = 0, one token past a group, 16 queries per wave
    (40, 40, 2, 32, 4, 1),       # T = n: the first query sees only token 0
    (2048, 256, 2, 128, 4, 1),   # several query blocks per stream
    (96, 7, 2, 128, 2, 0),       # everything in the residual window
    (1000, 100, 8, 128, 4, 1),   # 8-bit codes, causal
    (600, 16, 8, 64, 2, 0),      # 8-bit codes, split ranges
    # the workgroup layout follows T * GQ: one 16-column block per wavefront
    # below 128 columns, two from 128 on
    (900, 31, 2, 64, 4, 1),      # 124 columns: one block per wavefront
    (900, 32, 2, 64, 4, 1),      # 128 columns: two blocks per wavefront
    (1200, 70, 4, 128, 2, 0),    # two blocks per wavefront at GQ = 2
    (700, 130, 2, 32, 1, 1),     # two blocks per wavefront at GQ = 1, padding columns
])
def test_attn_shapes(orc, n, T, bits, R, gq, causal):
    _run(orc, 2, 2, 2 * gq, n, T, bits, R, causal, seed=n + T, label="attn-%d-%d" % (n, T))


def test_attn_chunked_prefill_and_fp32_queries(orc):
    """Chunks appended one after another (the cache streams), fp32 queries."""
    _run(orc, 1, 4, 16, 1500, 128, 2, 128, 1, seed=31, chunks=[1000, 372, 128],
         q_dtype=np.float32, label="chunked")


def test_attn_single_query_is_decode(orc):
    """One query without a mask agrees with the decode step (both against the
    oracle, and with each other to the tolerance)."""
    cache, q, out = _run(orc, 2, 8, 32, 3000, 1, 2, 128, 0, seed=41, label="T=1")
    dec = cache.decode(to_dev(np.ascontiguousarray(q[:, :, 0]))).cpu().numpy()
    assert rel_err(out[:, :, 0], dec) <= TOL


def test_attn_notebook_full_q(orc):
    """The notebook's attention over all 1024 rows of its Q (seed 1) on its
    fp32 cache (T=1024, D=128, no residual), 2-, 4- and 8-bit: parity with the
    oracle, and the notebook's own checks against unquantized attention."""
    import json, os
    import torch
    from kv_cache_quantization_amd import synth
    chk = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                      "notebook_checks.json")))["checks"]
    K, V, _ = synth.notebook_inputs()
    Q = torch.randn(1, 1024, 128, generator=torch.Generator().manual_seed(1)).numpy()
    q = Q.reshape(1, 1, 1024, 128).astype(np.float32)
    ref_fp = orc.attn_queries(q, K, V)
    rel = {}
    for bits in (2, 4, 8):
        cache = new_cache(1, 1, 1, 1024, bits=bits, R=0, dtype=np.float32)
        cache.append(to_dev(K), to_dev(V))
        out = cache.attn(to_dev(q)).cpu().numpy()
        c = orc.build_cache(K, V, bits, 32, 0)
        kh, vh = orc.dequant_cache(K, V, c)
        e = rel_err(out, orc.attn_queries(q, kh, vh))
        rel[bits] = np.linalg.norm(ref_fp - out) / np.linalg.norm(ref_fp)
        log("notebook full Q bits=%d: attn rel err %.3g, vs unquantized %.4f" % (bits, e, rel[bits]))
        assert e <= TOL
    assert rel[4] < chk["rel_err_4bit_max"]
    lo, hi = chk["rel_err_2bit_open_interval"]
    assert lo < rel[2] < hi


@pytest.mark.parametrize("n,T,bits,R,causal,chunks", [
    (1000, 100, 2, 128, 1, None),          # causal over codes and the residual
    (4096, 16, 4, 32, 0, None),            # split ranges + combine, 40 residual rows
    (96, 7, 2, 128, 0, None),              # everything in the residual
    (700, 64, 8, 64, 1, [500, 1] + [1] * 199),   # streamed: the ring wraps
])
def test_attn_fp32_cache_with_residual(orc, n, T, bits, R, causal, chunks):
    """A float32 cache whose residual holds tokens: its ring rows enter the
    attention's fp16 products rounded to nearest fp16; parity with the
    oracle's attention over the float32 rows themselves."""
    _run(orc, 2, 2, 8, n, T, bits, R, causal, seed=n + 7 * T, chunks=chunks,
         q_dtype=np.float32, dtype=np.float32, label="fp32-%d-%d" % (n, T))


def test_attn_errors():
    """Host-side checks: causal with more queries than tokens, an empty
    cache."""
    from kv_cache_quantization_amd import kivi, synth
    import torch
    cache = new_cache(1, 1, 4, 256, bits=2, R=32)
    q = torch.zeros((1, 4, 3, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(kivi.KiviError) as e:
        cache.attn(q)
    assert e.value.status == kivi.KIVI_ERR_STATE
    k, v = synth.kv_host(5, 1, 1, 2)
    cache.append(to_dev(k), to_dev(v))
    with pytest.raises(kivi.KiviError) as e:
        cache.attn(q, causal=True)                  # T = 3 > n = 2
    assert e.value.status == kivi.KIVI_ERR_INVALID_ARG


@pytest.mark.parametrize("G,bits,causal", [(64, 2, 1), (128, 4, 0)])
def test_group_sizes(orc, G, bits, causal):
    """G = 64 and 128 (the split layout): the stages take each block's codes,
    its key unit (one per key group) and its value pairs."""
    _run(orc, 2, 2, 8, 1111, 100, bits, 128, causal, seed=G + bits, label="attn-G%d" % G, G=G)


@pytest.mark.parametrize("G,causal", [(64, 1), (128, 0)])
def test_group_sizes_paper_policy(orc, G, causal):
    """The paper policy in the split layout: the last split's pass over the
    groups whose value codes stop at Q_V copies codes, key unit and value
    pairs into its stage (one-shot, and streamed across key flushes)."""
    _run(orc, 2, 2, 8, 1000, 300, 2, 128, causal, seed=G + 5, label="attn-paper-G%d" % G,
         G=G, policy=1)
    _run(orc, 1, 2, 8, 700, 40, 4, 128, causal, seed=G + 6, chunks=[500] + [1] * 200,
         label="attn-paper-stream-G%d" % G, G=G, policy=1)
