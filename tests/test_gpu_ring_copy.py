"""The copy of the newest rows into the residual ring takes one of four
routes under the window policy, and every route must leave the same ring
(and cache) as the oracle, bit for bit:

- folded into the quantize launch that reads only the appended chunk (a
  one-shot prefill, the chunks of 700, 300 and 257; a chunk whose flush also
  quantizes groups that start in the ring, which run in a launch of their own
  before it);
- folded into a quantize launch whose groups all read the ring, when the rows
  it reads and the rows the copy writes span less than the ring, so no slot
  is both (the last single-token step, which flushes a group);
- a ring-append launch after such a quantize launch when they span more (the
  chunk of 33);
- a ring-append launch alone (an append that quantizes nothing).

fp16 and fp32 rows (32 and 64 16-byte pieces per row pair), several streams
so that the copy workgroups cross stream boundaries, and G = 64 (key groups
of two blocks)."""
import numpy as np
import pytest

from gpu_helpers import check_cache, log, new_cache, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_quantization_amd import kivi
    kivi.lib()


@pytest.mark.parametrize("dtype,bits,R,group", [
    (np.float16, 2, 128, 32),
    (np.float32, 4, 64, 32),
    (np.float16, 8, 128, 64),
])
def test_ring_copy_routes(orc, dtype, bits, R, group):
    from kv_cache_quantization_amd import synth
    B, H, Hq = 3, 5, 10
    chunks = [700, 300, 1, 1, 5, 257, 33]
    # then enough rows that one more token ages a whole group out: that last
    # single-token step quantizes from the ring only
    m = 1
    while (sum(chunks) + m + 1 - R) % group:
        m += 1
    chunks += [m, 1]
    n = sum(chunks)
    k, v = synth.kv_host(90 + bits, B, H, n, dtype=dtype)
    cache = new_cache(B, H, Hq, n + 32, bits=bits, R=R, dtype=dtype, group=group)
    pos = 0
    for i, c in enumerate(chunks):
        before = cache.layout().n_quantized
        cache.append(to_dev(k[:, :, pos:pos + c]), to_dev(v[:, :, pos:pos + c]))
        pos += c
        lo = cache.layout()
        log("case ring-copy %s bits=%d R=%d G=%d: append %d -> n=%d, Q %d -> %d" %
            (np.dtype(dtype).name, bits, R, group, c, pos, before, lo.n_quantized))
        check_cache(orc, cache, k[:, :, :pos], v[:, :, :pos],
                    label="ring-copy-%d-%d" % (bits, i))
