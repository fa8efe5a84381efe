"""Pins of the oracle's KCVT mode (the GEAR review's "KCVT" section: keys per
channel with one group over all the tokens compressed together, values per
token with one group over the whole head dimension; "streaming buffer
strategy": new tokens wait in a full-precision buffer and are compressed
together when it fills).

Reading (segment policy): each flush quantizes one segment of tokens; a key
group is one channel of one segment, a value group one token's 128 channels;
Q(n) = n - (n mod R) with the buffer R a multiple of 32.

None of these re-types the oracle's arithmetic: they reduce KCVT to KIVI
configurations that tests/test_oracle_pins.py pins (segments of 32, 64 and
128 tokens are KIVI key groups of that size; values are KIVI value groups of
128 channels), check closed-form statistics of a whole-prefix segment
against numpy, check that a perturbation stays inside its (segment, channel)
group, and decode the packed blocks by the layout include/kivi.h documents.
"""
import numpy as np
import pytest

from test_oracle_layout_pins import decode_block_split, decode_kunit, documented_code_slots

D, T = 128, 32


def _kv(seed, B, H, n, dtype=np.float16):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, H, n, D)).astype(np.float32)
    v = rng.standard_normal((B, H, n, D)).astype(np.float32)
    k[:, :, :, [3, 17, 40, 88]] *= 5          # outlier key channels
    return k.astype(dtype), v.astype(dtype)


def test_segment_prefix_and_flush_schedule(orc):
    """Q(n) = n - (n mod R) for keys and values; a prefill of 300 tokens with
    R = 64 flushes [0, 256) as one segment, then every 64 single-token
    appends flush the 64 tokens that filled the buffer; deferred appends fold
    their rows into the next flush."""
    for n in (0, 1, 63, 64, 65, 300, 1000, 8704):
        assert orc.quantized_prefix(n, 32, 64, orc.POLICY_SEGMENT) == (n - n % 64,) * 2
    assert orc.segment_ends([300] + [1] * 150, 64) == [256, 320, 384, 448]
    assert orc.segment_ends([1000], 128) == [896]
    assert orc.segment_ends([40, 40, 40, 40], 64, deferred={1, 2}) == [128]
    assert orc.segment_ends([100, 40, 100], 32) == [96, 128, 224]


@pytest.mark.parametrize("seg", [32, 64, 128])
def test_equal_segments_are_kivi_groups(orc, seg):
    """Segments of `seg` tokens each give exactly the KIVI key groups of G =
    seg tokens (codes and fp16 zero / scale), and the values are KIVI value
    groups of G = 128 channels."""
    B, H, n = 1, 2, 512 + 40
    k, v = _kv(3 + seg, B, H, n)
    Q = 512
    kc = orc.build_cache(k, v, 2, D, 64, orc.POLICY_SEGMENT, segments=list(range(seg, Q + 1, seg)))
    kivi_k = orc.build_cache(k[:, :, :Q], v[:, :, :Q], 2, seg, 0)
    kivi_v = orc.build_cache(k[:, :, :Q], v[:, :, :Q], 2, D, 0)
    assert (kc["qk"], kc["qv"]) == (Q, Q)
    assert np.array_equal(kc["kcodes"], kivi_k["kcodes"])
    per = seg // T        # kcvt stores the pair per 32-token block
    assert np.array_equal(kc["kzero16"][:, :, ::per], kivi_k["kzero16"])
    assert np.array_equal(kc["kscale16"][:, :, ::per], kivi_k["kscale16"])
    assert np.array_equal(kc["vcodes"], kivi_v["vcodes"])
    assert np.array_equal(kc["vzero16"], kivi_v["vzero16"])
    assert np.array_equal(kc["vscale16"], kivi_v["vscale16"])


@pytest.mark.parametrize("bits", [2, 4])
def test_whole_prefix_segment_statistics(orc, bits):
    """One segment over the whole quantized prefix (a one-shot prefill): in
    every channel the zero is the fp16 input minimum over all Q tokens, the
    minimum element gets code 0 and the maximum the top level, every code
    lies in [0, 2^b - 1], and every reconstruction is within half a step
    plus the fp16 pair's rounding (the handbook's uniform-quantization
    bound)."""
    B, H, n, R = 1, 2, 1000, 128
    k, v = _kv(20 + bits, B, H, n)
    Q = n - n % R
    c = orc.build_cache(k, v, bits, D, R, orc.POLICY_SEGMENT, segments=[Q])
    L = (1 << bits) - 1
    kf = k.astype(np.float32)[:, :, :Q]
    kh, vh = orc.dequant_cache(k, v, c)
    for s in range(B * H):
        b, h = divmod(s, H)
        zmin = kf[b, h].min(0).astype(np.float16).view(np.uint16)
        for j in range(Q // T):
            assert np.array_equal(c["kzero16"][b, h, j], zmin)
            assert np.array_equal(c["kscale16"][b, h, j], c["kscale16"][b, h, 0])
        codes = c["kcodes"][b, h]
        assert codes.max() <= L
        assert (codes[kf[b, h].argmin(0), np.arange(D)] == 0).all()
        assert (codes[kf[b, h].argmax(0), np.arange(D)] == L).all()
        sf = c["kscale16"][b, h, 0].view(np.float16).astype(np.float64)
        zf = c["kzero16"][b, h, 0].view(np.float16).astype(np.float64)
        mn = kf[b, h].min(0).astype(np.float64)
        s_exact = (kf[b, h].max(0).astype(np.float64) - mn) / L
        bound = sf / 2 + L * np.abs(s_exact - sf) + np.abs(mn - zf) + 2.0 ** -20 * s_exact
        bound = bound + 2.0 ** -24 * (np.abs(kh[b, h, :Q]) + L * sf)
        assert (np.abs(kf[b, h] - kh[b, h, :Q]) <= bound * (1 + 2.0 ** -10) + 1e-30).all()
    # the residual stays verbatim
    assert np.array_equal(kh[:, :, Q:], k[:, :, Q:].astype(np.float32))
    assert np.array_equal(vh[:, :, Q:], v[:, :, Q:].astype(np.float32))


def test_segment_locality(orc):
    """One key outlier changes the codes and the pair of its own (segment,
    channel) group only, across that whole segment; values are untouched."""
    B, H, n = 1, 1, 448
    k, v = _kv(9, B, H, n, np.float32)
    segs = [256, 320, 384, 448]
    base = orc.build_cache(k, v, 2, D, 64, orc.POLICY_SEGMENT, segments=segs)
    t, ch = 300, 51                            # segment [256, 320)
    k2 = k.copy()
    k2[0, 0, t, ch] = 40.0
    pert = orc.build_cache(k2, v, 2, D, 64, orc.POLICY_SEGMENT, segments=segs)
    dk = np.argwhere(base["kcodes"][0, 0] != pert["kcodes"][0, 0])
    assert len(dk) > 0 and set(dk[:, 1]) == {ch}
    assert dk[:, 0].min() >= 256 and dk[:, 0].max() < 320
    assert dk[:, 0].min() < 256 + 16 and dk[:, 0].max() >= 320 - 16
    ds = np.argwhere(base["kscale16"][0, 0] != pert["kscale16"][0, 0])
    assert sorted(set(ds[:, 0])) == [8, 9] and set(ds[:, 1]) == {ch}
    assert np.array_equal(base["vcodes"], pert["vcodes"])


def test_packed_blocks_carry_their_segment(orc):
    """Packed by the layout include/kivi.h documents (the split layout: value
    groups span all 128 channels): each 32-token block holds its tokens' key
    codes and their one value pair each, and the block's key unit (one per
    32 tokens) holds the fp16 pair of the segment the block lies in."""
    B, H, n = 1, 2, 300
    k, v = _kv(31, B, H, n)
    segs = [128, 192, 256]
    c = orc.build_cache(k, v, 2, D, 64, orc.POLICY_SEGMENT, segments=segs)
    blocks, kside = orc.pack_cache(c)
    assert kside.shape == (B * H, 256 // T, 2, D)
    slots = documented_code_slots(2)
    for s in range(B * H):
        b, h = divmod(s, H)
        for j in range(256 // T):
            kc, vc, vs, vz = decode_block_split(blocks[s, j], 2, slots, 1)
            toks = slice(T * j, T * j + T)
            assert np.array_equal(kc, c["kcodes"][b, h, toks])
            assert np.array_equal(vc, c["vcodes"][b, h, toks])
            seg0 = [0] + segs
            i = next(i for i in range(len(segs)) if T * j < segs[i])
            first = seg0[i] // T             # the segment's first block shares the pair
            ks, kz = decode_kunit(kside[s, j])
            assert np.array_equal(ks, c["kscale16"][b, h, first])
            assert np.array_equal(kz, c["kzero16"][b, h, first])
            assert np.array_equal(vs[0], c["vscale16"][b, h, toks, 0])
            assert np.array_equal(vz[0], c["vzero16"][b, h, toks, 0])


def test_kcvt_attention_close_to_full_precision(orc):
    """Sanity of the whole path on the notebook-sized data at 4 bits (the
    review reports KCVT good at 4 bits, not at 2): decode attention over the
    dequantized KCVT cache stays close to attention over the fp16 cache,
    and 4 bits is closer than 2."""
    B, H, n = 1, 1, 1024
    k, v = _kv(40, B, H, n)
    rng = np.random.default_rng(41)
    q = rng.standard_normal((B, 4, D)).astype(np.float32)
    ref = orc.decode_attn(q, k.astype(np.float32), v.astype(np.float32))
    err = {}
    for bits in (2, 4):
        c = orc.build_cache(k, v, bits, D, 32, orc.POLICY_SEGMENT, segments=[1024])
        kh, vh = orc.dequant_cache(k, v, c)
        out = orc.decode_attn(q, kh, vh)
        err[bits] = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert err[4] < err[2] and err[4] < 0.2
