"""GPU parity at the full sizes of the serving workloads, in the launch
configuration the benchmark times.  Inputs are drawn on the device; a few
sampled streams are copied back and checked against the CPU oracle: packed
blocks, fp16 zero/scale, ring contents and (n, Q) bit for bit, and decode
attention of their query heads within the tolerance.

  * long context: batch 16 x 8 KV heads x 32 query heads, context 32768,
    2-bit, residual 128, one-shot prefill, one decode step;
  * streaming: batch 8, prefill 8192, then 512 single-token appends each
    followed by a decode step; the final cache equals a one-shot prefill of
    all 8704 tokens byte for byte (checked on the device for every stream);
  * capacity: batch 32, context 131072 appended in 8192-token chunks, 2- and
    4-bit, one decode step.
"""
import numpy as np
import pytest

from gpu_helpers import TOL, check_cache, log, oracle_decode, rel_err

pytestmark = pytest.mark.gpu

H, HQ, D, G = 8, 32, 128, 32
GQ = HQ // H


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_quantization_amd import kivi
    kivi.lib()
    yield
    torch.cuda.empty_cache()


def _check_streams(orc, cache, ks, vs, q, out, sample, bits, R, label):
    """ks, vs: {(b, h): [n, D] host arrays}; q, out: host [B, Hq, D]."""
    H_ = cache.cfg.n_kv_heads
    streams = [b * H_ + h for b, h in sample]
    k = np.stack([ks[s] for s in sample])
    v = np.stack([vs[s] for s in sample])
    check_cache(orc, cache, k, v, streams=streams, label=label)
    for i, (b, h) in enumerate(sample):
        qs = q[b, GQ * h:GQ * (h + 1)][None]
        ref = oracle_decode(orc, k[i][None, None], v[i][None, None], qs, bits, G, R)
        e = rel_err(out[b, GQ * h:GQ * (h + 1)], ref[0])
        log("  %s stream (%d, %d): decode rel err %.3g" % (label, b, h, e))
        assert e <= TOL, (label, b, h, e)


def test_long_context_b16():
    import torch
    from kv_cache_quantization_amd import KiviCache, synth
    import oracle as orc
    B, n, R, bits = 16, 32768, 128, 2
    log("case long-context B=%d n=%d" % (B, n))
    k, v = synth.kv_device(3, B, H, n)
    q = synth.queries_device(3, B, HQ)
    cache = KiviCache(B, H, HQ, n, bits=bits, residual=R, device="cuda:0")
    cache.append(k, v)
    out = cache.decode(q).cpu().numpy()
    sample = [(0, 0), (7, 3), (15, 7)]
    ks = {s: k[s].cpu().numpy() for s in sample}
    vs = {s: v[s].cpu().numpy() for s in sample}
    del k, v
    _check_streams(orc, cache, ks, vs, q.cpu().numpy(), out, sample, bits, R, "long-context")


def test_streaming_8192_plus_512():
    import torch
    from kv_cache_quantization_amd import KiviCache, synth
    import oracle as orc
    B, P, S, R, bits = 8, 8192, 512, 128, 2
    log("case streaming B=%d prefill=%d steps=%d" % (B, P, S))
    sample = [(0, 0), (5, 6)]
    k0, v0 = synth.kv_device(4, B, H, P, chunk=0)
    cache = KiviCache(B, H, HQ, P + S, bits=bits, residual=R, device="cuda:0")
    cache.append(k0, v0)
    ks, vs = [k0], [v0]
    hk = {s: [k0[s].cpu().numpy()] for s in sample}
    hv = {s: [v0[s].cpu().numpy()] for s in sample}
    check_at = {0, 31, 32, 255, S - 1}
    for s in range(S):
        k1, v1 = synth.kv_device(4, B, H, 1, chunk=1 + s)
        cache.append(k1, v1)
        ks.append(k1)
        vs.append(v1)
        for st in sample:
            hk[st].append(k1[st].cpu().numpy())
            hv[st].append(v1[st].cpu().numpy())
        q = synth.queries_device(4, B, HQ, step=s)
        out = cache.decode(q)
        if s in check_at:
            kk = {st: np.concatenate(hk[st]) for st in sample}
            vv = {st: np.concatenate(hv[st]) for st in sample}
            _check_streams(orc, cache, kk, vv, q.cpu().numpy(), out.cpu().numpy(), sample,
                           bits, R, "streaming step %d" % s)
    # the streamed cache equals a one-shot prefill of all P + S tokens
    kall, vall = torch.cat(ks, dim=2), torch.cat(vs, dim=2)
    one = KiviCache(B, H, HQ, P + S, bits=bits, residual=R, device="cuda:0")
    one.append(kall, vall)
    la, lb = cache.layout(), one.layout()
    assert (la.n_tokens, la.n_quantized) == (lb.n_tokens, lb.n_quantized) == (P + S, 8576)
    ng = la.n_quantized // G
    assert torch.equal(cache.blocks_view()[:, :ng], one.blocks_view()[:, :ng])
    slots = [t % la.ring_capacity for t in range(la.n_quantized, la.n_tokens)]
    for ra, rb in zip(cache.ring_views(), one.ring_views()):
        ra = ra.reshape(B * H, la.ring_capacity, D)[:, slots]
        rb = rb.reshape(B * H, la.ring_capacity, D)[:, slots]
        assert torch.equal(ra.view(torch.int16), rb.view(torch.int16))
    log("  streaming cache == one-shot cache (all %d streams)" % (B * H))


@pytest.mark.parametrize("bits", [2, 4])
def test_capacity_b32_131072_chunked(bits):
    import torch
    from kv_cache_quantization_amd import KiviCache, synth
    import oracle as orc
    B, n, C, R = 32, 131072, 8192, 128
    log("case capacity B=%d n=%d chunk=%d bits=%d" % (B, n, C, bits))
    sample = [(0, 0), (31, 7)]
    cache = KiviCache(B, H, HQ, n, bits=bits, residual=R, device="cuda:0")
    hk = {s: [] for s in sample}
    hv = {s: [] for s in sample}
    for ci in range(n // C):
        k, v = synth.kv_device(5, B, H, C, chunk=ci)
        cache.append(k, v)
        for s in sample:
            hk[s].append(k[s].cpu().numpy())
            hv[s].append(v[s].cpu().numpy())
        del k, v
    q = synth.queries_device(5, B, HQ)
    out = cache.decode(q).cpu().numpy()
    kk = {s: np.concatenate(hk[s]) for s in sample}
    vv = {s: np.concatenate(hv[s]) for s in sample}
    _check_streams(orc, cache, kk, vv, q.cpu().numpy(), out, sample, bits, R,
                   "capacity-%d" % bits)
    del cache
    torch.cuda.empty_cache()


def test_attn_long_context_b16():
    """Attention of T = 256 causal queries (a chunked-prefill step) and of 16
    unmasked queries over the long-context cache (batch 16, context 32768,
    2-bit, residual 128), in the launch configuration the benchmark times.
    Sampled streams and query rows are checked against the oracle: causal row
    t is the decode step over the first n - T + t + 1 dequantized tokens."""
    import torch
    from kv_cache_quantization_amd import KiviCache, synth
    import oracle as orc
    B, n, R, bits = 16, 32768, 128, 2
    log("case attn long-context B=%d n=%d" % (B, n))
    k, v = synth.kv_device(3, B, H, n)
    cache = KiviCache(B, H, HQ, n, bits=bits, residual=R, device="cuda:0")
    cache.append(k, v)
    sample = [(0, 0), (15, 7)]
    ks = {s: k[s].cpu().numpy() for s in sample}
    vs = {s: v[s].cpu().numpy() for s in sample}
    del k, v
    for T, causal, rows in ((256, True, (0, 100, 255)), (16, False, (0, 15))):
        qm = synth.queries_multi_device(3, B, HQ, T)
        out = cache.attn(qm, causal=causal).cpu().numpy()
        qh = qm.cpu().numpy()
        assert np.isfinite(out).all()
        for (b, h) in sample:
            ref_c = orc.build_cache(ks[(b, h)][None, None], vs[(b, h)][None, None], bits, G, R)
            kh, vh = orc.dequant_cache(ks[(b, h)][None, None], vs[(b, h)][None, None], ref_c)
            for t in rows:
                seen = n - T + t + 1 if causal else n
                q1 = qh[b, GQ * h:GQ * (h + 1), t][None]
                ref = orc.decode_attn(q1, kh[:, :, :seen], vh[:, :, :seen])
                e = rel_err(out[b, GQ * h:GQ * (h + 1), t], ref[0])
                log("  T=%d causal=%d stream (%d, %d) row %d: rel err %.3g" % (T, causal, b, h, t, e))
                assert e <= TOL, (T, causal, b, h, t, e)
    del cache
    torch.cuda.empty_cache()
