"""The fused path under HIP graph capture: its calls make no host read, no
allocation and no memset inside a step, so one step can be captured once
and replayed.  Every replay is checked against the CPU oracle element by
element, with eager work on the same outputs (fills) and an unrelated eager
pipeline run between the replays."""
import pytest

import oracle
import torch  # imported at collection so that its first-load time is not charged to a test
from gpu_util import compare, require_gpu, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("variant", ["two calls", "one call", "one pass"])
@pytest.mark.parametrize("wid,scale", [(1, 0.3), (3, 0.002)])
def test_fused_step_replays_from_a_graph(variant, wid, scale):
    import merge_front_coded_amd as em
    Ah, Bh = workload(wid, scale)
    ref = oracle.run(Ah, Bh, items_per_part=512)
    A, B = em.DeviceSide.from_host(Ah), em.DeviceSide.from_host(Bh)
    kw = {"one_call": variant == "one call", "one_pass": variant == "one pass"}
    pl = em.Pipeline(A, B, items_per_part=512, path="fused", **kw)
    # an unrelated pipeline whose eager runs are interleaved with the replays
    Oh, Ph = workload(1, 0.1)
    other = em.Pipeline(em.DeviceSide.from_host(Oh), em.DeviceSide.from_host(Ph), path="fused")
    print(f"graph replay {variant} workload {wid}@{scale}", flush=True)
    pl.run()
    compare(pl, ref, Ah, Bh, label=f"{variant}: eager")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pl.run(read_counts=False)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pl.run(read_counts=False)
    torch.cuda.synchronize()

    outs = [pl.payload, pl.final, pl.ord_A, pl.ord_B, pl.len_bits, pl.lcp, pl.off, pl.d_S, pl.d_T]
    for rep in range(3):
        for t in outs:
            t.fill_(-1 if rep % 2 else 0)
        other.run()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        pl.read_counts()
        compare(pl, ref, Ah, Bh, label=f"{variant}: replay {rep}")
