"""Pins of the oracle's packers (oracle_pack_blocks_kv in both layouts with
the split layout's key units, oracle_pack_outlier_records) against the byte
layout that include/kivi.h documents.

The decoders below are written from that documented layout alone, in the
forward direction (from a dword, a bit and a lane to the logical token and
channel).  They never call the oracle's code_position, whose search the packer
uses, so a wrong placement inside the packer cannot cancel out.  The logical
arrays they are compared with come from oracle_build_cache, which
tests/test_oracle_pins.py pins to the pages ([NB] "Asymmetric 2-bit
quantiser", [RV] 1.1 worked example and 3.2.3 Algorithm 1).

The storage cost is fixed by the notebook's storage cell (b bits per code and
two fp16 per group); the bit order is a layout choice of this library.
"""
import numpy as np
import pytest

D = 128
T = 32          # tokens per block


def documented_code_slots(bits):
    """Every code slot of one code area, from include/kivi.h's formula: for
    lane l (0..63), lane dword w (0..2b-1), half h and slot i (0..16/b-1),
    dword (w/4)*256 + 4l + w%4 holds at bits [16h + b i, +b) the code of
    operand o at position kk, where o = w*(4/b) + i/4 and kk = 2(i%4) + h
    for b = 2, 4, and o = w/2, kk = 4(w%2) + 2i + h for b = 8.  Keys: token
    16(o/4) + l%16, channel 32(o%4) + 8(l/16) + kk.  Values: channel
    16o + l%16, token 4(l/16) + kk%4 + 16(kk/4).
    Returns arrays (dword, shift, key_token, key_channel, val_token, val_channel)."""
    rows = []
    for l in range(64):
        for w in range(2 * bits):
            for h in range(2):
                for i in range(16 // bits):
                    if bits == 8:
                        o, kk = w // 2, 4 * (w % 2) + 2 * i + h
                    else:
                        o, kk = w * (4 // bits) + i // 4, 2 * (i % 4) + h
                    dword = (w // 4) * 256 + 4 * l + w % 4
                    shift = 16 * h + bits * i
                    kt, kc = 16 * (o // 4) + l % 16, 32 * (o % 4) + 8 * (l // 16) + kk
                    vc, vt = 16 * o + l % 16, 4 * (l // 16) + kk % 4 + 16 * (kk // 4)
                    rows.append((dword, shift, kt, kc, vt, vc))
    return tuple(np.array(c, dtype=np.int64) for c in zip(*rows))


def decode_code_area(area, bits, is_v, slots):
    """Codes [32 tokens][128 channels] of one code area (bytes) by the
    documented formula."""
    dword, shift, kt, kc, vt, vc = slots
    words = np.frombuffer(area.tobytes(), dtype="<u4").astype(np.int64)
    codes = (words[dword] >> shift) & ((1 << bits) - 1)
    out = np.full((T, D), -1, np.int64)
    tok, ch = (vt, vc) if is_v else (kt, kc)
    out[tok, ch] = codes
    return out


def decode_block(blk, bits, slots):
    """(kcodes, vcodes, kscale, kzero, vscale[4][32], vzero[4][32]) of one
    block, by the documented offsets: K codes, V codes (b*32*128/8 bytes
    each), then fp16 K scale[128], K zero[128], V scale[4][32], V zero[4][32]."""
    cb = bits * T * D // 8
    kc = decode_code_area(blk[:cb], bits, False, slots)
    vc = decode_code_area(blk[cb:2 * cb], bits, True, slots)
    side = np.frombuffer(blk[2 * cb:].tobytes(), dtype="<u2")
    assert side.size == 4 * D
    return kc, vc, side[:D], side[D:2 * D], side[2 * D:3 * D].reshape(4, T), \
        side[3 * D:].reshape(4, T)


def decode_block_split(blk, bits, slots, nvg):
    """(kcodes, vcodes, vscale[nvg][32], vzero[nvg][32]) of one block of the
    split layout (value groups of 128 / nvg channels > 32), by the
    documented offsets: K codes, V codes, then fp16 V scale[nvg][32], V
    zero[nvg][32] (slot gv of token t: value group gv)."""
    cb = bits * T * D // 8
    kc = decode_code_area(blk[:cb], bits, False, slots)
    vc = decode_code_area(blk[cb:2 * cb], bits, True, slots)
    side = np.frombuffer(blk[2 * cb:].tobytes(), dtype="<u2")
    assert side.size == 2 * nvg * T
    return kc, vc, side[:nvg * T].reshape(nvg, T), side[nvg * T:].reshape(nvg, T)


def decode_kunit(unit):
    """(kscale[128], kzero[128]) of one key unit of the split layout: fp16
    K scale[D], then K zero[D] (unit given as 512 bytes or [2][D] uint16)."""
    u = np.frombuffer(np.ascontiguousarray(unit).tobytes(), dtype="<u2")
    assert u.size == 2 * D
    return u[:D], u[D:]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_documented_layout_covers_every_code_once(bits):
    """The documented formula alone: every (token, channel) of a tile gets
    exactly one slot, slots do not overlap, and the area is b*32*128/8 bytes."""
    dword, shift, kt, kc, vt, vc = documented_code_slots(bits)
    n_dw = bits * T * D // 32
    assert dword.min() == 0 and dword.max() == n_dw - 1
    assert ((shift % bits) == 0).all() and shift.max() + bits <= 32
    assert len(set(zip(dword.tolist(), shift.tolist()))) == T * D
    for tok, ch in ((kt, kc), (vt, vc)):
        assert len(set(zip(tok.tolist(), ch.tolist()))) == T * D
        assert tok.min() == 0 and tok.max() == T - 1 and ch.min() == 0 and ch.max() == D - 1


@pytest.mark.parametrize("bits,G", [(2, 32), (4, 32), (8, 32), (2, 64), (4, 64), (2, 128),
                                    (8, 128)])
def test_pack_blocks_decode_to_logical_cache(orc, bits, G):
    """Window policy: every block decodes (documented formula and offsets) to
    the logical codes of its 32 tokens.  G = 32: the block carries the fp16
    zero / scale of its key group and, per value slot cg, the zero / scale
    of the value group holding channels 32cg .. 32cg + 31.  G = 64, 128 (the
    split layout): the block carries its tokens' 128 / G value pairs, slot gv
    of token t the pair of value group gv, and key unit u the zero / scale
    of key group u, once."""
    rng = np.random.default_rng(100 + bits + G)
    B, H, n, R = 1, 2, 5 * 64 + 17, G
    k = rng.standard_normal((B, H, n, D)).astype(np.float16)
    v = rng.standard_normal((B, H, n, D)).astype(np.float16)
    k[:, :, :, 5] *= 5
    c = orc.build_cache(k, v, bits, G, R)
    q = c["qk"]
    assert q == c["qv"] and q % G == 0 and q > 0
    blocks, kside = orc.pack_cache(c)
    nvg = D // G
    side_bytes = 4 * D * 2 if G == 32 else 2 * 2 * T * nvg
    assert blocks.shape == (B * H, q // T, 2 * bits * T * D // 8 + side_bytes)
    assert (kside is None) == (G == 32)
    if G > 32:
        assert kside.shape == (B * H, q // G, 2, D)
    slots = documented_code_slots(bits)
    for s in range(B * H):
        b, h = divmod(s, H)
        for j in range(q // T):
            toks = slice(T * j, T * j + T)
            if G == 32:
                kc, vc, ks, kz, vs, vz = decode_block(blocks[s, j], bits, slots)
                assert np.array_equal(ks, c["kscale16"][b, h, j])
                assert np.array_equal(kz, c["kzero16"][b, h, j])
                for cg in range(4):
                    assert np.array_equal(vs[cg], c["vscale16"][b, h, toks, cg])
                    assert np.array_equal(vz[cg], c["vzero16"][b, h, toks, cg])
            else:
                kc, vc, vs, vz = decode_block_split(blocks[s, j], bits, slots, nvg)
                for gv in range(nvg):
                    assert np.array_equal(vs[gv], c["vscale16"][b, h, toks, gv])
                    assert np.array_equal(vz[gv], c["vzero16"][b, h, toks, gv])
            assert np.array_equal(kc, c["kcodes"][b, h, toks])
            assert np.array_equal(vc, c["vcodes"][b, h, toks])
        if G > 32:
            for u in range(q // G):
                ks, kz = decode_kunit(kside[s, u])
                assert np.array_equal(ks, c["kscale16"][b, h, u])
                assert np.array_equal(kz, c["kzero16"][b, h, u])


@pytest.mark.parametrize("bits,G", [(2, 32), (2, 64), (4, 128), (8, 64)])
def test_packed_bytes_are_the_storage_cost(orc, bits, G):
    """The notebook's storage cell counts b bits per code and two fp16 per
    group.  In the split layout (G > 32) the packed bytes of Q tokens are
    exactly that, keys and values: Q*D*b/8 * 2 + 2*2*(Q/G*D + Q*D/G).  At
    G = 32 too (key groups per 32 tokens, value groups per 32 channels)."""
    rng = np.random.default_rng(5 + G + bits)
    n = 4 * 128 + 40
    k = rng.standard_normal((1, 1, n, D)).astype(np.float16)
    v = rng.standard_normal((1, 1, n, D)).astype(np.float16)
    c = orc.build_cache(k, v, bits, G, 0)
    Q = c["qk"]
    blocks, kside = orc.pack_cache(c)
    total = blocks.nbytes + (kside.nbytes if kside is not None else 0)
    codes = Q * D * bits // 8 * 2
    groups = Q // G * D + Q * D // G         # key groups + value groups
    assert total == codes + 2 * 2 * groups


def _pack_prefilled(orc, c, fill):
    """oracle_pack_blocks_kv into a buffer pre-filled with `fill`, so that
    bytes the packer must leave alone can be seen."""
    B, H, qk, qv, bits = c["B"], c["H"], c["qk"], c["qv"], c["bits"]
    ng = max(qk // T, -(-qv // T))
    G = c["G"]
    out = np.full((B * H, ng, orc.block_bytes(bits, G)), fill, np.uint8)
    nku = qk // G + 1
    kside = np.full((B * H, nku, 2, D), fill * 0x101, np.uint16) if G > 32 else None
    orc.lib().oracle_pack_blocks_kv(B, H, G, qk, qv, bits, ng, nku if G > 32 else 0,
                                    orc._p(c["kcodes"]), orc._p(c["kzero16"]),
                                    orc._p(c["kscale16"]), orc._p(c["vcodes"]),
                                    orc._p(c["vzero16"]), orc._p(c["vscale16"]), orc._p(out),
                                    orc._p(kside) if kside is not None else None)
    return (out, kside) if G > 32 else out


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_blocks_paper_policy_partial_value_block(orc, bits):
    """[RV] 3.2.3 Algorithm 1 (paper policy): keys quantized up to Q_K = n -
    n mod R, values up to Q_V = n - R.  Reading R4: inside the 32-token block
    holding Q_V, value rows at or past Q_V pack as code 0 with zero / scale
    0; blocks past the value prefix keep their value area untouched; key
    areas of all Q_K / 32 blocks hold the key codes."""
    rng = np.random.default_rng(7 + bits)
    B, H, R, G = 1, 2, 64, 32
    n = 150                                  # Q_K = 128, Q_V = 86: block 2 holds rows 64..95
    k = rng.standard_normal((B, H, n, D)).astype(np.float16)
    v = rng.standard_normal((B, H, n, D)).astype(np.float16)
    c = orc.build_cache(k, v, bits, G, R, policy=orc.POLICY_PAPER)
    assert (c["qk"], c["qv"]) == (128, 86)
    out = _pack_prefilled(orc, c, 0xAB)
    slots = documented_code_slots(bits)
    cb = bits * T * D // 8
    for s in range(B * H):
        b, h = divmod(s, H)
        for j in range(4):
            kc, vc, ks, kz, vs, vz = decode_block(out[s, j], bits, slots)
            toks = slice(T * j, T * j + T)
            assert np.array_equal(kc, c["kcodes"][b, h, toks])
            assert np.array_equal(ks, c["kscale16"][b, h, j])
            assert np.array_equal(kz, c["kzero16"][b, h, j])
            if j == 3:
                # no value row of this block is quantized: untouched
                assert (out[s, j, cb:2 * cb] == 0xAB).all()
                assert (out[s, j, 2 * cb + 2 * 2 * D:] == 0xAB).all()
                continue
            lim = min(T, c["qv"] - T * j)       # 32, 32, 22
            assert np.array_equal(vc[:lim], c["vcodes"][b, h, T * j:T * j + lim])
            assert (vc[lim:] == 0).all()
            for cg in range(4):
                assert np.array_equal(vs[cg, :lim], c["vscale16"][b, h, T * j:T * j + lim, cg])
                assert np.array_equal(vz[cg, :lim], c["vzero16"][b, h, T * j:T * j + lim, cg])
                assert (vs[cg, lim:] == 0).all() and (vz[cg, lim:] == 0).all()
    # the zero rows really are a departure from the values: the same rows of
    # a fully quantized cache are not all-zero
    full = orc.build_cache(k, v, bits, G, 0, policy=orc.POLICY_WINDOW)
    assert (full["vcodes"][:, :, 86:96] != 0).any()


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_blocks_paper_policy_split_layout(orc, bits):
    """The paper policy at G = 64 (split layout): keys quantized up to Q_K =
    n - n mod R, values up to Q_V = n - R (R4: rows at or past Q_V inside
    the block holding it pack as code 0 with zero / scale 0; blocks past
    the value prefix keep their value area, key units past Q_K / G stay
    untouched)."""
    rng = np.random.default_rng(70 + bits)
    B, H, R, G = 1, 2, 64, 64
    n = 230                                  # Q_K = 192, Q_V = 166: block 5 holds rows 160..191
    k = rng.standard_normal((B, H, n, D)).astype(np.float16)
    v = rng.standard_normal((B, H, n, D)).astype(np.float16)
    c = orc.build_cache(k, v, bits, G, R, policy=orc.POLICY_PAPER)
    assert (c["qk"], c["qv"]) == (192, 166)
    out, kside = _pack_prefilled(orc, c, 0xAB)
    assert out.shape[1] == 6 and kside.shape[1] == 4
    slots = documented_code_slots(bits)
    nvg = D // G
    for s in range(B * H):
        b, h = divmod(s, H)
        for j in range(6):
            kc, vc, vs, vz = decode_block_split(out[s, j], bits, slots, nvg)
            toks = slice(T * j, T * j + T)
            assert np.array_equal(kc, c["kcodes"][b, h, toks])
            lim = min(T, c["qv"] - T * j)       # 32 ... 32, then 6
            assert np.array_equal(vc[:lim], c["vcodes"][b, h, T * j:T * j + lim])
            assert (vc[lim:] == 0).all()
            for gv in range(nvg):
                assert np.array_equal(vs[gv, :lim], c["vscale16"][b, h, T * j:T * j + lim, gv])
                assert np.array_equal(vz[gv, :lim], c["vzero16"][b, h, T * j:T * j + lim, gv])
                assert (vs[gv, lim:] == 0).all() and (vz[gv, lim:] == 0).all()
        for u in range(3):
            ks, kz = decode_kunit(kside[s, u])
            assert np.array_equal(ks, c["kscale16"][b, h, u])
            assert np.array_equal(kz, c["kzero16"][b, h, u])
        assert (kside[s, 3] == 0xABAB).all()


@pytest.mark.parametrize("n_out", [1, 2, 3])
def test_outlier_records_documented_layout(orc, n_out):
    """Records decoded by include/kivi.h's offsets: uint16 channel[3] at byte
    0 (ascending, 0xFFFF when unused), zero bytes 6..15, fp16 values [3][32]
    at byte 16 + 64 o (0 when unused), zero bytes 208..255.  The channels are a brute-force top-n
    of max |K| over the key group's tokens (ties: the lower channel), and the
    values the fp16 inputs themselves -- neither taken from the oracle."""
    rng = np.random.default_rng(40 + n_out)
    B, H, n, G = 2, 2, 4 * 32 + 9, 32
    k = rng.standard_normal((B, H, n, D)).astype(np.float16)
    v = rng.standard_normal((B, H, n, D)).astype(np.float16)
    k[1, 0, 33, 64] = 8.0              # a tie in group 1 of stream 2
    k[1, 0, 40, 12] = -8.0
    c = orc.build_cache(k, v, 2, G, 0, key_outliers=n_out)
    ng = c["qk"] // G
    rec = orc.pack_outlier_records(c, ng + 1)
    rec[:, ng] = 0x5A                  # past the prefix: must be left alone
    rec2 = np.full_like(rec, 0x5A)
    orc.lib().oracle_pack_outlier_records(B, H, c["qk"], n_out, ng + 1, orc._p(c["kout_idx"]),
                                          orc._p(c["kout_val"]), orc._p(rec2))
    assert (rec2[:, ng] == 0x5A).all()
    kf = k.astype(np.float32)
    for s in range(B * H):
        b, h = divmod(s, H)
        for j in range(ng):
            r = rec2[s, j]
            idx = np.frombuffer(r[:6].tobytes(), dtype="<u2")
            assert (r[6:16] == 0).all()
            vals = np.frombuffer(r[16:208].tobytes(), dtype="<u2").reshape(3, 32)
            assert (r[208:] == 0).all()
            score = np.abs(kf[b, h, G * j:G * j + G]).max(0)
            want = sorted(sorted(range(D), key=lambda ch: (-score[ch], ch))[:n_out])
            assert list(idx[:n_out]) == want
            assert (idx[n_out:] == 0xFFFF).all()
            for o, ch in enumerate(want):
                assert np.array_equal(vals[o], k[b, h, G * j:G * j + G, ch].view(np.uint16))
            assert (vals[n_out:] == 0).all()
    # stream 2, group 1: channels 12 and 64 tie at |8|; one kept channel goes to 12
    kept = set(np.frombuffer(rec2[2, 1, :6].tobytes(), dtype="<u2")[:n_out].tolist())
    assert 12 in kept and (64 in kept) == (n_out >= 2)
