"""GPU parity at the full sizes of the serving workloads, in the launch
configuration the benchmark times.  Inputs are drawn on the device; sampled
streams (16 of them on the long-context and capacity workloads, spread over
batch entries and KV heads, the last stream included) are copied back and
checked against the CPU oracle: packed blocks, fp16 zero/scale, outlier
records, ring contents and (n, Q) bit for bit, and decode attention of their
query heads within the tolerance.  The oracle work of the sampled streams
runs on a thread pool (its C calls release the interpreter lock).

  * long context: batch 16 x 8 KV heads x 32 query heads, context 32768,
    residual 128, one-shot prefill, one decode step -- at 2, 4 and 8 bits,
    at 2 bits with two fp16 key channels per key group, and in the split
    layout at G = 64 (2-bit) and G = 128 (4-bit);
  * streaming: batch 8, prefill 8192, then 512 single-token appends each
    followed by a decode step, under the window policy and under the review's
    Algorithm-1 policy (key flushes every 128 steps); the final cache equals
    a one-shot prefill of all 8704 tokens byte for byte (checked on the
    device for every stream);
  * capacity: batch 32, context 131072 appended in 8192-token chunks, 2- and
    4-bit, one decode step.
"""
from concurrent.futures import ThreadPoolExecutor

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


def spread_sample(B, n=16):
    """n (batch, KV head) streams spread over batch entries and heads, the
    last stream (B-1, H-1) included."""
    picks = [((i * B) // n, (3 * i + 1) % H) for i in range(n - 1)] + [(B - 1, H - 1)]
    assert len(set(picks)) == n
    return picks


class StreamSnapshot:
    """Host copy of one stream of a cache, presented as a one-stream cache
    to gpu_helpers.check_cache (blocks, outlier records and ring rows of
    stream (b, h) only)."""

    def __init__(self, cache, b, h):
        import torch
        torch.cuda.synchronize()
        s = b * cache.cfg.n_kv_heads + h
        self.cfg = cache.cfg
        self._lo = cache.layout()
        self._blocks = cache.blocks_view()[s:s + 1].cpu()
        self._rec = cache.outlier_records_view()[s:s + 1].cpu() if cache.cfg.key_outliers else None
        ks = cache.kside_view()
        self._ks = ks[s:s + 1].cpu() if ks is not None else None
        rk, rv = cache.ring_views()
        self._ring = (rk[b:b + 1, h:h + 1].cpu(), rv[b:b + 1, h:h + 1].cpu())

    def layout(self):
        return self._lo

    def blocks_view(self):
        return self._blocks

    def outlier_records_view(self):
        return self._rec

    def kside_view(self):
        return self._ks

    def ring_views(self):
        return self._ring


def _check_streams(orc, cache, ks, vs, q, out, sample, bits, R, label, policy=0, n_out=0,
                   group=G):
    """ks, vs: {(b, h): [n, D] host arrays}; q, out: host [B, Hq, D]."""
    snaps = {s: StreamSnapshot(cache, *s) for s in sample}

    def one(s):
        b, h = s
        k, v = ks[s][None], vs[s][None]
        check_cache(orc, snaps[s], k, v, streams=[0], label="%s (%d, %d)" % (label, b, h))
        qs = q[b, GQ * h:GQ * (h + 1)][None]
        ref = oracle_decode(orc, k[None], v[None], qs, bits, group, R, policy=policy,
                            key_outliers=n_out)
        return rel_err(out[b, GQ * h:GQ * (h + 1)], ref[0])

    with ThreadPoolExecutor(max_workers=16) as ex:
        errs = list(ex.map(one, sample))
    worst = max(errs)
    log("  %s: %d streams bit-exact, decode rel err max %.3g" % (label, len(sample), worst))
    for s, e in zip(sample, errs):
        assert e <= TOL, (label, s, e)


@pytest.mark.parametrize("bits,n_out,group", [(2, 0, 32), (4, 0, 32), (8, 0, 32), (2, 2, 32),
                                              (2, 0, 64), (4, 0, 128)])
def test_long_context_b16(bits, n_out, group):
    """G = 64 and 128 run the split layout (key units once per group): the
    key units of the sampled streams are compared bit for bit too."""
    import torch
    from kv_cache_quantization_amd import KiviCache, synth
    import oracle as orc
    B, n, R = 16, 32768, 128
    log("case long-context B=%d n=%d bits=%d key_outliers=%d G=%d" % (B, n, bits, n_out, group))
    k, v = synth.kv_device(3, B, H, n)
    q = synth.queries_device(3, B, HQ)
    cache = KiviCache(B, H, HQ, n, bits=bits, group=group, residual=R, device="cuda:0",
                      key_outliers=n_out)
    cache.append(k, v)
    out = cache.decode(q).cpu().numpy()
    sample = spread_sample(B)
    ks = {s: k[s].cpu().numpy() for s in sample}
    vs = {s: v[s].cpu().numpy() for s in sample}
    del k, v
    _check_streams(orc, cache, ks, vs, q.cpu().numpy(), out, sample, bits, R,
                   "long-context %d-bit G=%d%s" % (bits, group, "" if not n_out else
                                                    ", %d kept" % n_out),
                   n_out=n_out, group=group)
    del cache
    torch.cuda.empty_cache()


@pytest.mark.parametrize("policy", [0, 1], ids=["window", "paper"])
def test_streaming_8192_plus_512(policy):
    """Under the paper policy the key residual is quantized 128 tokens at a
    time (steps 127, 255, 383 and 511 flush keys) and one value row per step;
    the checked steps include the first flush, the steps around it, and the
    last one."""
    import torch
    from kv_cache_quantization_amd import KiviCache, synth
    import oracle as orc
    B, P, S, R, bits = 8, 8192, 512, 128, 2
    log("case streaming B=%d prefill=%d steps=%d policy=%d" % (B, P, S, policy))
    sample = [(0, 0), (5, 6), (7, 7)]
    k0, v0 = synth.kv_device(4, B, H, P, chunk=0)
    cache = KiviCache(B, H, HQ, P + S, bits=bits, residual=R, device="cuda:0", policy=policy)
    cache.append(k0, v0)
    ks, vs = [k0], [v0]
    hk = {s: [k0[s].cpu().numpy()] for s in sample}
    hv = {s: [v0[s].cpu().numpy()] for s in sample}
    check_at = {0, 31, 32, 255, S - 1} if policy == 0 else {0, 126, 127, 128, 300, S - 1}
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
                           bits, R, "streaming step %d" % s, policy=policy)
    # the streamed cache equals a one-shot prefill of all P + S tokens
    kall, vall = torch.cat(ks, dim=2), torch.cat(vs, dim=2)
    one = KiviCache(B, H, HQ, P + S, bits=bits, residual=R, device="cuda:0", policy=policy)
    one.append(kall, vall)
    la, lb = cache.layout(), one.layout()
    want_q = (8576, 8576) if policy == 0 else (8704, 8576)
    assert (la.n_tokens, la.n_quantized, la.n_vquantized) == \
        (lb.n_tokens, lb.n_quantized, lb.n_vquantized) == (P + S,) + want_q
    # key parts of every block with key codes, whole blocks below Q_V (the
    # value areas past Q_V hold whatever the buffers held: under the paper
    # policy no value row of those blocks is quantized yet)
    ngk, ngv = la.n_quantized // G, la.n_vquantized // G
    cb = la.code_bytes
    kpart = list(range(cb)) + list(range(2 * cb, 2 * cb + 4 * D))
    assert torch.equal(cache.blocks_view()[:, :ngk, kpart], one.blocks_view()[:, :ngk, kpart])
    assert torch.equal(cache.blocks_view()[:, :ngv], one.blocks_view()[:, :ngv])
    for ra, rb, q0 in zip(cache.ring_views(), one.ring_views(),
                          (la.n_quantized, la.n_vquantized)):
        slots = [t % la.ring_capacity for t in range(q0, la.n_tokens)]
        if not slots:
            continue
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
    sample = spread_sample(B)
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
