"""GPU parity under the paper's flush policy ("[Paper review] KIVI ...",
3.2.2 and the prefill / decoding phases of Algorithm 1 in 3.2.3): keys are
quantized R tokens at a time (Q_K = n - n mod R), values one token at a time
(Q_V = max(0, n - R)).

Bit-exact against the oracle built under the same policy: key groups below
Q_K, value rows below Q_V (rows past Q_V in the group holding it are 0), the
ring contents, n, Q_K and Q_V.  Decode attention (split items over groups
with key and value codes, the item over the groups whose value codes stop
early, and the residual item) and the attention of T queries within 2e-3 of
the oracle's attention over the same dequantized cache.
"""
import numpy as np
import pytest

from gpu_helpers import TOL, check_cache, log, new_cache, oracle_decode, rel_err, to_dev

pytestmark = pytest.mark.gpu

PAPER = 1


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_quantization_amd import kivi
    kivi.lib()   # fail loudly if the HIP library is missing


def _run(orc, B, H, Hq, n, bits, R, seed, chunks=None, dtype=np.float16, q_dtype=np.float16,
         label=""):
    from kv_cache_quantization_amd import synth
    log("case %s: B=%d H=%d Hq=%d n=%d bits=%d R=%d %s chunks=%s" %
        (label, B, H, Hq, n, bits, R, np.dtype(dtype).name,
         chunks if chunks is None or len(chunks) < 12 else "%d chunks" % len(chunks)))
    k, v = synth.kv_host(seed, B, H, n, dtype=dtype)
    q = synth.queries_host(seed, B, Hq, dtype=q_dtype)
    cache = new_cache(B, H, Hq, max_tokens=n + 64, bits=bits, R=R, dtype=dtype, policy=PAPER)
    pos = 0
    for c in (chunks or [n]):
        cache.append(to_dev(k[:, :, pos:pos + c]), to_dev(v[:, :, pos:pos + c]))
        pos += c
    assert pos == n
    ref = check_cache(orc, cache, k, v, label=label)
    log("  Q_K=%d Q_V=%d" % (ref["qk"], ref["qv"]))
    out = cache.decode(to_dev(q)).cpu().numpy()
    want = oracle_decode(orc, k, v, q, bits, 32, R, policy=PAPER)
    e = rel_err(out, want)
    log("  decode rel err %.3g" % e)
    assert e <= TOL, (label, e)
    return cache


@pytest.mark.parametrize("n,bits,R,gq", [
    (10, 2, 32, 4),        # all residual (n < R)
    (64, 2, 64, 4),        # n = R: keys of all R quantized, values none
    (65, 2, 64, 4),        # one value row quantized (partial value group)
    (100, 4, 64, 2),       # key residual 36, value rows [0, 36)
    (1000, 2, 128, 4),     # Q_K = 896, Q_V = 872: three groups with early-stopping values
    (1024, 8, 128, 1),     # n a multiple of R: empty key residual
    (777, 4, 32, 4),       # R = G
    (2049, 2, 128, 2),
    (4613, 2, 2304, 4),    # Q_K = 4608, Q_V = 2309: 72 mixed groups, two per item
])
def test_oneshot(orc, n, bits, R, gq):
    _run(orc, 2, 3, 3 * gq, n, bits, R, seed=n + 7, label="paper-%d" % n)


def test_streaming_equals_oneshot(orc):
    """Under the paper policy too, any chunking gives the one-shot cache: keys
    move when n crosses a multiple of R, values one token per step."""
    rng = np.random.default_rng(1)
    n = 700
    chunks = [150] + [1] * 140 + [int(x) for x in rng.integers(1, 40, 12)]
    chunks.append(n - sum(chunks))
    assert chunks[-1] > 0
    for bits in (2, 4, 8):
        _run(orc, 2, 2, 8, n, bits, 64, seed=11, chunks=chunks, label="paper-stream-%d" % bits)


def test_token_by_token_decode_steps(orc):
    """Append one token, decode, for every step across two key flushes
    (decoding phase of Algorithm 1): the cache and each decode step match
    the oracle at every n."""
    from kv_cache_quantization_amd import synth
    B, H, Hq, R, bits = 1, 2, 8, 32, 2
    n0, steps = 90, 80
    k, v = synth.kv_host(31, B, H, n0 + steps)
    cache = new_cache(B, H, Hq, n0 + steps, bits=bits, R=R, policy=PAPER)
    cache.append(to_dev(k[:, :, :n0]), to_dev(v[:, :, :n0]))
    worst = 0.0
    for s in range(steps):
        n = n0 + s + 1
        cache.append(to_dev(k[:, :, n - 1:n]), to_dev(v[:, :, n - 1:n]))
        if s % 10 == 9 or n % R in (0, 1):
            check_cache(orc, cache, k[:, :, :n], v[:, :, :n], label="paper-step-%d" % n)
        q = synth.queries_host(1000 + s, B, Hq)
        out = cache.decode(to_dev(q)).cpu().numpy()
        e = rel_err(out, oracle_decode(orc, k[:, :, :n], v[:, :, :n], q, bits, 32, R,
                                       policy=PAPER))
        worst = max(worst, e)
        assert e <= TOL, (n, e)
    log("paper token-by-token: worst decode rel err %.3g" % worst)


def test_fp32_cache(orc):
    """float32 K/V rows (the residual and the early-stopping value rows come
    from a float32 ring), float32 queries."""
    _run(orc, 1, 2, 8, 300, 4, 64, seed=41, dtype=np.float32, q_dtype=np.float32,
         label="paper-fp32")
    _run(orc, 1, 2, 8, 300, 2, 64, seed=42, chunks=[200] + [1] * 100, dtype=np.float32,
         label="paper-fp32-stream")


def test_deferred_flush(orc):
    """KIVI_DEFER_FLUSH under the paper policy: rows wait in the ring (from the
    start of the value group holding Q_V) until flush(); the result equals
    the one-shot cache."""
    from kv_cache_quantization_amd import kivi, synth
    from kv_cache_quantization_amd import KiviError
    B, H, Hq, R, bits = 2, 2, 8, 64, 2
    n = 400
    k, v = synth.kv_host(51, B, H, n)
    cache = new_cache(B, H, Hq, n, bits=bits, R=R, policy=PAPER)
    cache.append(to_dev(k[:, :, :250]), to_dev(v[:, :, :250]))
    pos = 250
    while True:
        lo = cache.layout()
        room = lo.ring_capacity - (lo.n_tokens - lo.n_vquantized // 32 * 32)
        if room == 0:
            break
        c = min(room, 5)
        cache.append(to_dev(k[:, :, pos:pos + c]), to_dev(v[:, :, pos:pos + c]), defer_flush=True)
        pos += c
    with pytest.raises(KiviError) as e:
        cache.append(to_dev(k[:, :, pos:pos + 1]), to_dev(v[:, :, pos:pos + 1]), defer_flush=True)
    assert e.value.status == kivi.KIVI_ERR_CAPACITY
    with pytest.raises(KiviError) as e:
        cache.decode(to_dev(synth.queries_host(51, B, Hq)))
    assert e.value.status == kivi.KIVI_ERR_STATE
    cache.flush()
    cache.flush()
    check_cache(orc, cache, k[:, :, :pos], v[:, :, :pos], label="paper-deferred")
    cache.append(to_dev(k[:, :, pos:n]), to_dev(v[:, :, pos:n]))
    check_cache(orc, cache, k, v, label="paper-deferred-then-plain")
    q = synth.queries_host(52, B, Hq)
    out = cache.decode(to_dev(q)).cpu().numpy()
    e = rel_err(out, oracle_decode(orc, k, v, q, bits, 32, R, policy=PAPER))
    log("paper deferred: decode rel err %.3g" % e)
    assert e <= TOL


def _attn(orc, B, H, Hq, n, T, bits, R, causal, seed, chunks=None, label="",
          dtype=np.float16):
    from kv_cache_quantization_amd import kivi, synth
    k, v = synth.kv_host(seed, B, H, n, dtype=dtype)
    q = synth.queries_multi_host(seed, B, Hq, T)
    cache = new_cache(B, H, Hq, max_tokens=n + 64, bits=bits, R=R, policy=PAPER, dtype=dtype)
    pos = 0
    for c in (chunks or [n]):
        cache.append(to_dev(k[:, :, pos:pos + c]), to_dev(v[:, :, pos:pos + c]))
        pos += c
    lo = cache.layout()
    plan = kivi.kivi_attn_plan(cache.handle, T)
    log("case %s: B=%d H=%d Hq=%d n=%d T=%d bits=%d R=%d causal=%d Q_K=%d Q_V=%d plan=%s" %
        (label, B, H, Hq, n, T, bits, R, causal, lo.n_quantized, lo.n_vquantized, plan))
    out = cache.attn(to_dev(q), causal=causal).cpu().numpy()
    ref_cache = orc.build_cache(k, v, bits, 32, R, PAPER)
    kh, vh = orc.dequant_cache(k, v, ref_cache)
    e = rel_err(out, orc.attn_queries(q, kh, vh, causal))
    log("  attn rel err %.3g" % e)
    assert np.isfinite(out).all(), label
    assert e <= TOL, (label, e)


@pytest.mark.parametrize("n,T,bits,R,gq,causal", [
    (10, 4, 2, 32, 4, 0),        # all residual
    (65, 5, 2, 64, 4, 1),        # Q_K = 64, Q_V = 1: two groups of key codes, one value row
    (1000, 300, 2, 128, 4, 1),   # Q_K = 896, Q_V = 872: causal over codes, mixed group, ring
    (2049, 16, 2, 128, 2, 0),    # Q_K = 2048, Q_V = 1921: four mixed groups, split ranges
    (777, 33, 4, 32, 4, 0),      # R = G
    (1024, 64, 8, 128, 1, 1),    # n a multiple of R: empty key residual
])
def test_attn_queries(orc, n, T, bits, R, gq, causal):
    """The attention of T queries under the paper policy: groups with key and
    value codes in the split ranges, the groups whose value codes stop at
    Q_V (values from the ring above it) and the key residual [Q_K, n)."""
    _attn(orc, 2, 2, 2 * gq, n, T, bits, R, causal, seed=n + T, label="paper-attn-%d" % n)


def test_attn_queries_streamed_and_fp32(orc):
    """A streamed paper-policy cache (one-token appends across a key flush);
    float32 caches whose mixed groups take their value rows from the ring,
    one-shot and streamed."""
    _attn(orc, 1, 2, 8, 300, 40, 2, 64, 1, seed=71, chunks=[200] + [1] * 100,
          label="paper-attn-stream")
    _attn(orc, 1, 2, 8, 1000, 300, 2, 128, 1, seed=72, dtype=np.float32,
          label="paper-attn-fp32")
    _attn(orc, 1, 2, 8, 300, 40, 4, 64, 0, seed=73, chunks=[200] + [1] * 100,
          dtype=np.float32, label="paper-attn-fp32-stream")
