"""Decode steps captured in a HIP graph (as the streaming benchmark replays
them) give the eager results: single-token appends followed by decode
attention (two calls, or one kivi_append_decode) are captured once, then the
graph is replayed several times from a restored post-prefill cache, with the
program's own eager work and synchronizations between the replays.  Every
replay's decode outputs must equal the eager run's bit for bit, and its final
cache must match the oracle bit for bit, under both flush policies."""
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


@pytest.mark.parametrize("policy,fused", [(0, False), (1, False), (0, True)])
def test_graph_replays_equal_eager(orc, policy, fused):
    import torch
    from kv_cache_quantization_amd import synth
    B, H, Hq, R, bits, P, S = 2, 2, 8, 64, 2, 300, 70
    log("case graph policy=%d fused=%d prefill=%d steps=%d" % (policy, fused, P, S))
    k, v = synth.kv_host(71, B, H, P + S)
    kd, vd = to_dev(k), to_dev(v)
    rows = [(kd[:, :, P + s:P + s + 1].contiguous(), vd[:, :, P + s:P + s + 1].contiguous())
            for s in range(S)]
    qs = [to_dev(synth.queries_host(72, B, Hq, step=s)) for s in range(S)]
    outs = torch.empty((S, B, Hq, 128), dtype=torch.float32, device="cuda")

    cache = new_cache(B, H, Hq, P + S, bits=bits, R=R, policy=policy)
    cache.workspace()

    def prefill():
        cache.reset()
        cache.append(kd[:, :, :P].contiguous(), vd[:, :, :P].contiguous())

    def run_steps():
        for s in range(S):
            if fused:
                cache.append_decode(*rows[s], qs[s], out=outs[s])
            else:
                cache.append(*rows[s])
                cache.decode(qs[s], out=outs[s])

    prefill()
    run_steps()
    torch.cuda.synchronize()
    eager = outs.clone()
    check_cache(orc, cache, k, v, label="graph-eager")

    prefill()
    torch.cuda.synchronize()
    snap = cache.buffer.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        run_steps()
    torch.cuda.synchronize()
    for rep in range(3):
        cache.buffer.copy_(snap)
        outs.zero_()
        g.replay()
        torch.cuda.synchronize()
        x = torch.randn(1 << 20, device="cuda").sum()          # unrelated eager work
        torch.cuda.synchronize()
        assert torch.isfinite(x)
        assert torch.equal(outs, eager), "replay %d: decode outputs differ from the eager run" % rep
        check_cache(orc, cache, k, v, label="graph-replay-%d" % rep)
        log("  replay %d == eager" % rep)
