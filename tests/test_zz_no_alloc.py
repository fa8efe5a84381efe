"""kivi_decode_attn_noalloc (decode partials in the library's fixed device
array, no workspace argument) against kivi_decode_attn with a caller
workspace: the same kernels and plan, so the outputs must be identical bit for
bit, and both within the decode tolerance of the oracle.  Two calls in a row,
the second over a smaller cache, so that the second call finds the first
one's partials in the shared array."""
import numpy as np
import pytest

from gpu_helpers import TOL, log, new_cache, oracle_decode, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_quantization_amd import kivi
    kivi.lib()


def _one(orc, B, n, bits, R, policy, q_f32, seed):
    import torch
    from kv_cache_quantization_amd import kivi, synth
    H, Hq = 8, 32
    log("case noalloc: B=%d n=%d bits=%d R=%d policy=%d q_f32=%d" % (B, n, bits, R, policy, q_f32))
    k, v = synth.kv_host(seed, B, H, n)
    q = synth.queries_host(seed + 1, B, Hq, dtype=np.float32 if q_f32 else np.float16)
    cache = new_cache(B, H, Hq, n, bits=bits, R=R, policy=policy)
    cache.append(to_dev(k), to_dev(v))
    qd = to_dev(q)
    want = cache.decode(qd)
    got = torch.full_like(want, float("nan"))
    stream = torch.cuda.current_stream().cuda_stream
    qt = kivi.KIVI_F32 if q_f32 else kivi.KIVI_F16
    assert kivi.kivi_decode_workspace_bytes(cache.handle) <= kivi.KIVI_NOALLOC_SCRATCH_BYTES
    kivi.kivi_decode_attn_noalloc(cache.handle, qd.data_ptr(), qt, 0.0, got.data_ptr(), stream)
    torch.cuda.synchronize()
    assert torch.equal(got, want), "noalloc output differs from the workspace call"
    e = rel_err(got.cpu().numpy(), oracle_decode(orc, k, v, q, bits, 32, R, policy=policy))
    log("  equal to the workspace call; rel err vs oracle %.3g" % e)
    assert e <= TOL
    return cache


def test_noalloc_two_calls_second_smaller(orc):
    """First a batch-4 cache of 3000 tokens (2 bits, window policy), then a
    batch-2 cache of 700 tokens (4 bits, paper policy, fp32 queries) whose
    partials are fewer and land where the first call's were."""
    _one(orc, 4, 3000, 2, 128, 0, False, 10)
    _one(orc, 2, 700, 4, 64, 1, True, 20)

