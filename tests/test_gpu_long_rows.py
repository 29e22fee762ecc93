"""Selection on rows longer than 512 slices of 8192 keys (4,194,304 tokens).

The final order-statistic kernel then covers the slices' counts and the answer digit's
candidate segments in more than one pass of its 256 threads.  No K or V is needed: ts_select
takes scores, and ts_score_select reads only the 32-wide index.  Parity follows the staged rules
of test_gpu_parity: scores within the fp32 bound, theta the exact order statistic of the GPU
scores, votes and lists bit-exact against the oracle on the GPU's scores and votes.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

from gpu_util import bits, dev, f64, score_bound, to_dev

pytestmark = pytest.mark.gpu

N = 4_400_000          # 538 slices of 8192 keys, 538 slices of 128 tiles in the fused path


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def check_selection(sel, s64, offsets, mode):
    idx = sel["idx"].cpu().numpy()
    if mode == api.MODE_VOTE:
        th = O.theta(s64, offsets, 9, 10)
        assert np.array_equal(f64(sel["theta"]), th), "theta is not the order statistic of the scores"
        v = O.votes(s64, th, offsets)
        assert np.array_equal(sel["votes"].cpu().numpy().astype(np.int32), v), "votes differ"
        ref, _ = O.select_vote(v, offsets, 1, 5)
    else:
        ref, _ = O.select_per_head(s64, offsets, 1, 5)
    assert np.array_equal(idx, ref), "selection differs from the oracle"


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_select_on_long_rows(mode):
    rng = np.random.default_rng(23)
    offsets = np.array([0, N], np.int64)
    offs = api.Offsets(offsets, dev())
    sc = np.zeros((2, api.score_stride(offs)), np.float32)
    sc[:, :N] = rng.standard_normal((2, N), dtype=np.float32)
    vote = mode == api.MODE_VOTE
    sel = api.select(to_dev(sc), offs, 1, api.params(mode, (1, 5)), want_theta=vote, want_votes=vote)
    torch.cuda.synchronize()
    check_selection(sel, sc[:, :N].astype(np.float64), offsets, mode)


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_score_select_on_long_rows(mode):
    rng = np.random.default_rng(29)
    offsets = np.array([0, N], np.int64)
    P = synth.projection(rng)
    q = synth.normal_bf16(rng, (1, 2, 128))
    kidx = synth.normal_bf16(rng, (N, 1, 32))
    offs = api.Offsets(offsets, dev())
    p = api.params(mode, (1, 5))
    vote = mode == api.MODE_VOTE
    qd, Pd, kd = to_dev(q), to_dev(P), to_dev(kidx)
    fused = api.score_select(qd, Pd, kd, offs, 1, p, want_theta=vote, want_votes=vote)
    sc = api.score(qd, Pd, kd, offs, 1)
    calls = api.select(sc, offs, 1, p, want_theta=vote, want_votes=vote)
    torch.cuda.synchronize()
    assert torch.equal(fused["scores"][:, :N], sc[:, :N]), "fused scores differ from ts_score"
    for k in ("idx", "count") + (("theta", "votes") if vote else ()):
        assert torch.equal(fused[k], calls[k]), f"fused {k} differs from ts_select"
    s64 = f64(fused["scores"])[:, :N]
    ref = O.score(q, P, bits(kd), offsets, 2, 1)
    assert not (np.abs(s64 - ref) > 2 * score_bound(q, P, kidx, offsets, 2, 1) + 1e-30).any()
    check_selection(fused, s64, offsets, mode)
