"""The segment policy (KCVT: the GEAR review's coarse-grained grouping with
its streaming buffer) on the GPU against the oracle: packed blocks, fp16
zero/scale, ring contents and (n, Q) bit for bit, decode attention and the
attention of several queries within the tolerance.

Each flush of the full-precision buffer (Q(n) = n - n mod R) quantizes one
segment: one zero / scale per key channel over the whole segment (a
one-shot prefill is one segment), one per token over all 128 value
channels.  The oracle is told the flush segments (oracle.segment_ends of
the same append sequence)."""
import numpy as np
import pytest

from gpu_helpers import TOL, check_cache, log, new_cache, oracle_decode, rel_err, to_dev

pytestmark = pytest.mark.gpu

SEG = 2          # KIVI_FLUSH_SEGMENT


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_quantization_amd import kivi
    kivi.lib()
    yield
    torch.cuda.empty_cache()


def _decode_check(orc, cache, k, v, q, segs, label):
    out = cache.decode(to_dev(q)).cpu().numpy()
    c = cache.cfg
    ref = oracle_decode(orc, k, v, q, c.bits, 128, c.residual, policy=SEG, segments=segs)
    e = rel_err(out, ref)
    log("  %s: decode rel err %.3g" % (label, e))
    assert e <= TOL, (label, e)


@pytest.mark.parametrize("bits,dtype,gq", [(2, np.float16, 4), (4, np.float16, 4),
                                           (8, np.float16, 2), (2, np.float32, 1)])
def test_one_shot_prefill_is_one_segment(orc, bits, dtype, gq):
    """A prefill of 1000 tokens with a 64-token buffer quantizes [0, 960) as
    one segment (keys: one pair per channel over 960 tokens) and keeps 40
    tokens in the buffer."""
    import torch
    from kv_cache_quantization_amd import synth
    B, H, n, R = 2, 8, 1000, 64
    log("case kcvt one-shot bits=%d %s gq=%d" % (bits, np.dtype(dtype).name, gq))
    k, v = synth.kv_host(31, B, H, n, dtype=dtype)
    q = synth.queries_host(32, B, H * gq, dtype=np.float16)
    cache = new_cache(B, H, H * gq, n, bits=bits, R=R, dtype=dtype, policy=SEG, group=128)
    cache.append(to_dev(k), to_dev(v))
    segs = orc.segment_ends([n], R)
    assert segs == [960]
    check_cache(orc, cache, k, v, label="one-shot", segments=segs)
    _decode_check(orc, cache, k, v, q, segs, "one-shot")
    if dtype == np.float16:
        # the attention of several queries reads the same blocks
        T = 16
        qm = synth.queries_multi_host(33, B, H * gq, T)
        out = cache.attn(to_dev(qm), causal=True).cpu().numpy()
        ref_c = orc.build_cache(k, v, bits, 128, R, SEG, segments=segs)
        kh, vh = orc.dequant_cache(k, v, ref_c)
        ref = orc.attn_queries(qm, kh, vh, causal=True)
        e = rel_err(out, ref)
        log("  one-shot attention of %d causal queries: rel err %.3g" % (T, e))
        assert e <= TOL
    del cache
    torch.cuda.empty_cache()


def test_streaming_flushes_one_segment_per_buffer(orc):
    """Prefill 300 (segment [0, 256)), then 150 single-token appends with a
    decode step each: the buffer of 64 tokens flushes [256, 320), [320, 384)
    and [384, 448) as segments of their own; cache and decode checked at
    every flush step and the steps around it."""
    from kv_cache_quantization_amd import synth
    B, H, Hq, P, S, R, bits = 2, 8, 32, 300, 150, 64, 2
    log("case kcvt streaming prefill=%d steps=%d R=%d" % (P, S, R))
    n = P + S
    k, v = synth.kv_host(41, B, H, n)
    cache = new_cache(B, H, Hq, n, bits=bits, R=R, policy=SEG, group=128)
    cache.append(to_dev(k[:, :, :P]), to_dev(v[:, :, :P]))
    pos, appends = P, [P]
    check_at = {0, 18, 19, 20, 83, 84, 148, 149}
    for s in range(S):
        cache.append(to_dev(k[:, :, pos:pos + 1]), to_dev(v[:, :, pos:pos + 1]))
        pos += 1
        appends.append(1)
        if s in check_at:
            segs = orc.segment_ends(appends, R)
            kk, vv = k[:, :, :pos], v[:, :, :pos]
            check_cache(orc, cache, kk, vv, label="step %d" % s, segments=segs)
            q = synth.queries_host(42, B, Hq, step=s)
            _decode_check(orc, cache, kk, vv, q, segs, "step %d (segments %s)" % (s, segs))
    assert orc.segment_ends(appends, R) == [256, 320, 384, 448]


def test_chunks_deferred_flush_and_errors(orc):
    """Appends of several sizes, some deferred (rows buffered only) and then
    folded into the next flush, and an explicit kivi_flush: each flush is
    one segment.  Decode refuses a cache whose deferred rows have filled the
    buffer (a flush pending) and accepts one whose buffer is not full."""
    from kv_cache_quantization_amd import kivi, synth
    B, H, Hq, R, bits = 2, 8, 32, 96, 4
    sizes = [130, 50, 20, 40, 7, 200, 33]
    deferred = {1, 2, 4}
    n = sum(sizes)
    log("case kcvt chunks %s deferred %s R=%d" % (sizes, sorted(deferred), R))
    k, v = synth.kv_host(51, B, H, n, dtype=np.float16)
    cache = new_cache(B, H, Hq, n, bits=bits, R=R, policy=SEG, group=128)
    pos, done = 0, []
    for i, m in enumerate(sizes):
        cache.append(to_dev(k[:, :, pos:pos + m]), to_dev(v[:, :, pos:pos + m]),
                     defer_flush=i in deferred)
        pos += m
        done.append(m)
        if i in deferred:
            lo = cache.layout()
            if orc.quantized_prefix(pos, 32, R, orc.POLICY_SEGMENT)[0] > lo.n_quantized:
                with pytest.raises(kivi.KiviError) as e:
                    cache.decode(to_dev(synth.queries_host(52, B, Hq)))
                assert e.value.status == kivi.KIVI_ERR_STATE
            continue
        segs = orc.segment_ends(done, R, deferred=deferred)
        check_cache(orc, cache, k[:, :, :pos], v[:, :, :pos], label="after append %d" % i,
                    segments=segs)
        _decode_check(orc, cache, k[:, :, :pos], v[:, :, :pos],
                      synth.queries_host(53, B, Hq, step=i), segs, "append %d" % i)
    # a deferred append that fills the buffer, then kivi_flush
    extra = 100
    k2, v2 = synth.kv_host(54, B, H, extra, dtype=np.float16)
    big = new_cache(B, H, Hq, n + extra, bits=bits, R=R, policy=SEG, group=128)
    big.append(to_dev(k), to_dev(v))
    big.append(to_dev(k2), to_dev(v2), defer_flush=True)
    big.flush()
    kk, vv = np.concatenate([k, k2], 2), np.concatenate([v, v2], 2)
    segs = orc.segment_ends([n, extra], R)
    assert segs == [480, 576]
    check_cache(orc, big, kk, vv, label="flush", segments=segs)


def test_long_segment_b4_32768(orc):
    """A one-shot prefill of 32768 tokens (+ 40 in the buffer) is one
    segment of 1024 blocks: its statistics pass runs over 64 chunks per
    stream; sampled streams bit-exact and decode within tolerance."""
    import torch
    from kv_cache_quantization_amd import KiviCache, synth
    B, H, Hq, n, R, bits = 4, 8, 32, 32768 + 40, 128, 2
    log("case kcvt long segment B=%d n=%d" % (B, n))
    k, v = synth.kv_device(3, B, H, n)
    q = synth.queries_device(3, B, Hq)
    cache = KiviCache(B, H, Hq, n, bits=bits, group=128, residual=R, device="cuda:0",
                      policy=SEG)
    cache.append(k, v)
    out = cache.decode(q).cpu().numpy()
    segs = orc.segment_ends([n], R)
    assert segs == [32768]
    qh = q.cpu().numpy()
    for b, h in ((0, 0), (3, 7), (1, 5)):
        s = b * H + h
        kk, vv = k[b, h].cpu().numpy(), v[b, h].cpu().numpy()
        check_cache(orc, cache, kk[None], vv[None], streams=[s], label="stream %d" % s,
                    segments=segs)
        ref = oracle_decode(orc, kk[None, None], vv[None, None], qh[b, 4 * h:4 * h + 4][None],
                            bits, 128, R, policy=SEG, segments=segs)
        e = rel_err(out[b, 4 * h:4 * h + 4], ref[0])
        log("  stream (%d, %d): decode rel err %.3g" % (b, h, e))
        assert e <= TOL
    del cache
    torch.cuda.empty_cache()
