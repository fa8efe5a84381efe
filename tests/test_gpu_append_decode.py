"""kivi_append_decode (append, then one decode step, in one call) against
kivi_append followed by kivi_decode_attn on a second cache fed the same rows:
decode outputs bit-identical at every step, and both caches bit-exact against
the oracle.  When nothing ages out of the residual, the fused call's decode
reads the new rows from the caller's buffer and writes them into the ring
itself; flush steps and the paper policy take the two-call route."""
import numpy as np
import pytest

from gpu_helpers import TOL, check_cache, log, new_cache, oracle_decode, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_quantization_amd import kivi
    kivi.lib()


def _loop(orc, B, H, Hq, P, steps, bits, R, dtype=np.float16, policy=0, step_sizes=None,
          q_dtype=np.float16, seed=0, label=""):
    import torch
    from kv_cache_quantization_amd import synth
    sizes = step_sizes or [1] * steps
    n = P + sum(sizes)
    log("case %s: B=%d H=%d Hq=%d prefill=%d steps=%d bits=%d R=%d %s policy=%d" %
        (label, B, H, Hq, P, len(sizes), bits, R, np.dtype(dtype).name, policy))
    k, v = synth.kv_host(seed, B, H, n, dtype=dtype)
    fused = new_cache(B, H, Hq, n, bits=bits, R=R, dtype=dtype, policy=policy)
    split = new_cache(B, H, Hq, n, bits=bits, R=R, dtype=dtype, policy=policy)
    for c in (fused, split):
        c.append(to_dev(k[:, :, :P]), to_dev(v[:, :, :P]))
    pos, worst = P, 0.0
    for s, m in enumerate(sizes):
        kd, vd = to_dev(k[:, :, pos:pos + m]), to_dev(v[:, :, pos:pos + m])
        q = synth.queries_host(seed + 1, B, Hq, step=s, dtype=q_dtype)
        qd = to_dev(q)
        a = fused.append_decode(kd, vd, qd)
        split.append(kd, vd)
        b = split.decode(qd)
        pos += m
        torch.cuda.synchronize()
        assert torch.equal(a, b), "%s step %d: fused and two-call outputs differ" % (label, s)
        if s % 16 == 15 or s == len(sizes) - 1:
            e = rel_err(a.cpu().numpy(), oracle_decode(orc, k[:, :, :pos], v[:, :, :pos], q, bits,
                                                       32, R, policy=policy))
            worst = max(worst, e)
            assert e <= TOL, (label, s, e)
    check_cache(orc, fused, k, v, label=label + "-fused")
    check_cache(orc, split, k, v, label=label + "-split")
    log("  %d steps equal, worst decode rel err %.3g" % (len(sizes), worst))


@pytest.mark.parametrize("bits,R,gq", [(2, 128, 4), (4, 64, 2), (8, 32, 1), (2, 0, 4)])
def test_fused_equals_two_calls(orc, bits, R, gq):
    """Single-token steps across several group flushes (every 32nd step
    quantizes a group: the two-call route; the others are fused)."""
    _loop(orc, 2, 2, 2 * gq, 300, 80, bits, R, seed=bits + R, label="fused-%d-%d" % (bits, R))


def test_fused_multi_token_and_fp32(orc):
    """Appends of 3 and 5 tokens that stay in the residual; a float32 cache
    (the residual items' float32 path reads and writes the new rows too)."""
    _loop(orc, 2, 2, 8, 200, 0, 2, 128, step_sizes=[3, 5, 1, 3, 5, 2, 7, 1, 4, 6] * 3, seed=3,
          label="fused-multi")
    _loop(orc, 1, 2, 8, 150, 40, 4, 64, dtype=np.float32, q_dtype=np.float32, seed=4,
          label="fused-fp32")


def test_paper_policy_takes_two_calls(orc):
    _loop(orc, 2, 2, 8, 150, 40, 2, 64, policy=1, seed=5, label="fused-paper")


def test_errors_leave_cache_unchanged(orc):
    import torch
    from kv_cache_quantization_amd import kivi, synth
    from kv_cache_quantization_amd import KiviError
    k, v = synth.kv_host(6, 1, 1, 140)
    c = new_cache(1, 1, 4, 256, bits=2, R=64)
    c.append(to_dev(k[:, :, :100]), to_dev(v[:, :, :100]))
    q = to_dev(synth.queries_host(6, 1, 4))
    # deferred rows up to n = 128: Q(128) = 64 > Q(100) = 32, a flush is pending
    c.append(to_dev(k[:, :, 100:128]), to_dev(v[:, :, 100:128]), defer_flush=True)
    assert (c.layout().n_tokens, c.layout().n_quantized) == (128, 32)
    with pytest.raises(KiviError) as e:           # deferred flush pending
        c.append_decode(to_dev(k[:, :, 128:129]), to_dev(v[:, :, 128:129]), q)
    assert e.value.status == kivi.KIVI_ERR_STATE
    c.flush()
    out = torch.empty((1, 4, 128), dtype=torch.float32, device="cuda")
    ws = c.workspace()
    k1, v1 = to_dev(k[:, :, 128:129]), to_dev(v[:, :, 128:129])
    with pytest.raises(KiviError) as e:           # workspace too small
        kivi.kivi_append_decode(c.handle, k1.data_ptr(), v1.data_ptr(), 1, q.data_ptr(), 0, 0.0,
                                out.data_ptr(), ws.data_ptr(), 16, 0)
    assert e.value.status == kivi.KIVI_ERR_BUFFER_TOO_SMALL
    with pytest.raises(KiviError) as e:           # bad query dtype
        kivi.kivi_append_decode(c.handle, k1.data_ptr(), v1.data_ptr(), 1, q.data_ptr(), 9, 0.0,
                                out.data_ptr(), ws.data_ptr(), ws.numel(), 0)
    assert e.value.status == kivi.KIVI_ERR_INVALID_ARG
    with pytest.raises(KiviError) as e:           # over capacity
        kivi.kivi_append_decode(c.handle, k1.data_ptr(), v1.data_ptr(), 200, q.data_ptr(), 0,
                                0.0, out.data_ptr(), ws.data_ptr(), ws.numel(), 0)
    assert e.value.status == kivi.KIVI_ERR_CAPACITY
    assert (c.layout().n_tokens, c.layout().n_quantized) == (128, 64)   # no effect
    check_cache(orc, c, k[:, :, :128], v[:, :, :128], label="fused-errors")
    c.append_decode(k1, v1, q)                    # and a good call afterwards
    check_cache(orc, c, k[:, :, :129], v[:, :, :129], label="fused-after-errors")
