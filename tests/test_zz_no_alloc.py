"""em_scan_noalloc, the scan for callers that cannot allocate: its look-back
state lives in a fixed device array of the library instead of a caller
workspace.  Its offsets must equal em_scan's, bit for bit, on consecutive
calls that share that array (the second smaller than the first, then an empty
one), and a size beyond its limit is rejected before any work."""
import numpy as np
import pytest
import torch

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _lengths(n, seed):
    # record lengths in bits, up to 2^20, so that the offsets pass 2^32
    return np.random.default_rng(seed).integers(0, 1 << 20, n, dtype=np.uint32)


def test_noalloc_scan_matches_em_scan_on_consecutive_calls():
    import merge_front_coded_amd as em
    for n, seed in ((3_000_001, 11), (70_001, 12), (4096, 13), (0, 14)):
        print(f"scan of {n} lengths (seed {seed})", flush=True)
        host = _lengths(n, seed)
        lens = torch.from_numpy(host.view(np.int32)).cuda() if n else torch.zeros(4, dtype=torch.int32,
                                                                                    device="cuda")
        want = torch.full((n + 1,), -1, dtype=torch.int64, device="cuda")
        got = torch.full((n + 1,), -2, dtype=torch.int64, device="cuda")
        ws = torch.empty(max(em.em_workspace_bytes(n, 0, 256), 256), dtype=torch.uint8, device="cuda")
        em.em_scan(lens, n, want, ws)
        em.em_scan_noalloc(lens, n, got)
        torch.cuda.synchronize()
        g = got.cpu().numpy().view(np.uint64)
        w = want.cpu().numpy().view(np.uint64)
        bad = np.nonzero(g != w)[0]
        assert bad.size == 0, f"n={n}: offsets differ from em_scan at {bad[:5]}"
        ref = np.zeros(n + 1, np.uint64)
        np.cumsum(host.astype(np.uint64), out=ref[1:])
        assert np.array_equal(g, ref), f"n={n}: offsets differ from the prefix sums"


def test_noalloc_scan_rejects_sizes_beyond_its_array():
    import merge_front_coded_amd as em
    lens = torch.zeros(16, dtype=torch.int32, device="cuda")
    off = torch.zeros(16, dtype=torch.int64, device="cuda")
    with pytest.raises(em.EmError) as e:
        em.em_scan_noalloc(lens, em.binding.EM_MAX_RECORDS, off)
    assert e.value.code == em.binding.EM_ERANGE
