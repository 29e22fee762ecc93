"""ts_sparse_decode_timed: the same result as ts_sparse_decode, bit for bit, plus the gather
kernel's duration from its dispatch timestamps (positive, and below the event time of the whole
call, which adds the merge kernel and the launch gaps)."""
import numpy as np
import pytest
import torch

from query_aware_sparse_index_amd import api, synth

from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_timed_decode_matches(mode):
    x = synth.make_decode(2, [30000, 5000], 32, 8, 8, False)
    rng = np.random.default_rng(11 + mode)
    lists, counts = [], []
    for b in range(2):
        n = int(x.offsets[b + 1] - x.offsets[b])
        k = n // 5
        counts.append(k)
        for _ in range(1 if mode == api.MODE_VOTE else 32):
            lists.append(np.sort(rng.choice(n, size=k, replace=False)).astype(np.int32))
    offs = api.Offsets(x.offsets, dev())
    q, K, V = to_dev(x.q), to_dev(x.K), to_dev(x.V)
    idx = to_dev(np.concatenate(lists))
    cd = torch.tensor(counts, dtype=torch.int64, device=dev())
    ref = api.sparse_decode(q, K, V, offs, idx, cd, counts, mode)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    out, us = api.sparse_decode_timed(q, K, V, offs, idx, cd, counts, mode)
    b.record()
    torch.cuda.synchronize()
    call_us = a.elapsed_time(b) * 1e3
    print(f"mode {mode}: gather {us:.1f} us, call {call_us:.1f} us", flush=True)
    assert torch.equal(out, ref), "the timed call changes the result"
    assert 0 < us < call_us
