"""GPU parity of the HIP path against the fp64 CPU oracle (staged).

Rules (each stage is compared on the GPU's own inputs to that stage, so that legal fp32
vs fp64 near-ties cannot cascade):
  * index append: the GPU index equals the oracle's bf16 values bit for bit (both sum the
    fp64 products in the same order and round once);
  * scores: |gpu - oracle(gpu index)| <= 2 x the fp32 dot-product error bound;
  * theta: the exact nearest-rank order statistic of the GPU scores;
  * votes and selections: bit-exact against the oracle run on the GPU scores / votes;
  * decode: max abs error <= 2e-3 against the oracle run on the GPU index lists.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

from gpu_util import Step, bits, check_staged, dev, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def test_c1_vote_step():
    r = check_staged(Step(synth.config1()).run())
    print("c1 vote", r)


def test_c1_per_head_step():
    r = check_staged(Step(synth.config1(), mode=api.MODE_PER_HEAD).run())
    print("c1 per-head", r)


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_c2_step(mode):
    r = check_staged(Step(synth.config2(), mode=mode).run())
    print("c2", mode, r)


@pytest.mark.parametrize("lengths,budget", [([5000, 1234, 300, 4097], (3, 20)), ([70000, 20000], (1, 5))])
@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_ragged_batch(lengths, budget, mode):
    x = synth.make_decode(4, lengths, 32, 8, lambda n: n // 100, False, budget, 3)
    check_staged(Step(x, mode=mode).run())


# every (Hkv, G) pair the library instantiates, a ragged two-sequence batch that spans
# several 512-token score blocks and ends in partial blocks
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (2, 1), (4, 1), (8, 1), (2, 2), (4, 2), (8, 2), (16, 2), (4, 4), (8, 4),
                                    (16, 4), (32, 4), (8, 8), (16, 8), (32, 8), (64, 8)])
@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_head_layouts(Hq, Hkv, mode):
    x = synth.make_decode(4, [1537, 700], Hq, Hkv, 8, False, (1, 5), 11)
    check_staged(Step(x, mode=mode, local=64).run())


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_full_budget_equals_dense(mode):
    x = synth.make_decode(1, [3000], 8, 2, 16, False, (1, 1), 5)
    st = Step(x, mode=mode).run()
    idx = st.sel["idx"].cpu().numpy()
    reps = 1 if mode == api.MODE_VOTE else 8
    assert np.array_equal(idx, np.tile(np.arange(3000), reps))
    dense = api.dense_decode(st.q, st.K, st.V, st.offs)
    torch.cuda.synchronize()
    ref = O.dense_decode(x.q, x.K, x.V, x.offsets, 8, 2)
    assert np.abs(f64(dense) - ref).max() <= 2e-3
    assert np.abs(f64(st.out) - ref).max() <= 2e-3


def test_short_sequences_take_everything():
    for n in (1, 5, 259, 260, 261):
        x = synth.make_decode(1, [n], 8, 2, 0, False, (1, 10), n)
        st = Step(x).run()
        k = O.budget_tokens(n, 1, 10, 4, 256)
        idx = st.sel["idx"].cpu().numpy()
        assert len(idx) == k
        if n <= 260:
            assert np.array_equal(idx, np.arange(n))
        check_staged(st)


def test_zero_query_ties_to_lowest_positions():
    x = synth.make_decode(1, [5000], 8, 2, 0, False, (1, 10), 2)
    x.q[:] = 0
    for mode in (api.MODE_VOTE, api.MODE_PER_HEAD):
        st = Step(x, mode=mode).run()
        assert np.all(f64(st.scores)[:, :5000] == 0)
        check_staged(st)
        idx = st.sel["idx"].cpu().numpy()[:500]
        assert np.array_equal(idx, np.r_[0:244, 4744:5000])


# rows longer than the LDS candidate capacity whose threshold sits in a mass of equal
# scores: the sampled bracket collapses onto the tied key and the final kernel falls back
# to the whole-row radix select
@pytest.mark.parametrize("zero_frac", [1.0, 0.95])
def test_heavy_ties_long_rows(zero_frac):
    x = synth.make_decode(1, [40000], 8, 2, 0, False, (1, 5), 6)
    nz = int(40000 * zero_frac)
    rng = np.random.default_rng(6)
    rows = rng.permutation(40000)[:nz]
    x.K[rows] = 0                     # zero keys -> zero index rows -> scores exactly 0
    for mode in (api.MODE_VOTE, api.MODE_PER_HEAD):
        st = Step(x, mode=mode).run()
        check_staged(st)


# a row longer than one tile of the vote scan (256 chunks of 1024 tokens) and longer than
# the LDS candidate capacity of the threshold select
@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_long_row(mode):
    x = synth.make_decode(3, [300000], 8, 2, 300, False, (1, 5), 9)
    check_staged(Step(x, mode=mode).run())


def test_median_threshold_and_vmin():
    x = synth.config1()
    check_staged(Step(x, theta=(1, 2)).run())
    check_staged(Step(x, vmin=3).run())
    check_staged(Step(x, sink=0, local=0).run())


def test_incremental_append_equals_batch_build():
    x = synth.config1()
    n = 4096
    K = to_dev(x.K)
    P = to_dev(x.P)
    a = torch.empty((n, 2, 32), dtype=torch.int16, device=dev())
    b = torch.empty_like(a)
    api.index_append(K, P, a, 0)
    api.index_append(K[:4000], P, b, 0)
    for t in range(4000, n):
        api.index_append(K[t:t + 1], P, b, t)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_repeat_is_deterministic():
    x = synth.config2()
    s1 = Step(x).run()
    s2 = Step(x).run()
    assert torch.equal(s1.scores, s2.scores)
    assert torch.equal(s1.sel["idx"], s2.sel["idx"])
    assert torch.equal(s1.out, s2.out)


def test_dense_decode_c2():
    x = synth.config2()
    q, K, V = to_dev(x.q), to_dev(x.K), to_dev(x.V)
    out = api.dense_decode(q, K, V, api.Offsets(x.offsets, dev()))
    torch.cuda.synchronize()
    ref = O.dense_decode(x.q, x.K, x.V, x.offsets, 32, 8)
    assert np.abs(f64(out) - ref).max() <= 2e-3


def test_error_codes_on_device_calls():
    x = synth.config1()
    st = Step(x)
    with pytest.raises(api.QasiError) as e:
        api.score(st.q[:, :6].contiguous(), st.P, torch.empty((4096, 2, 32), dtype=torch.int16, device=dev()), st.offs, 4)
    assert e.value.code in (-1, -2)
    with pytest.raises(api.QasiError) as e:
        api.snapkv_compress(st.q[:1], st.K, st.V, 64, pool_kernel=5)
    assert e.value.code == -2


# the hand-worked vote example (tests/golden/vote_worked_example.txt) fed straight to
# ts_select; a fourth all-zero head (theta 0, no strict votes) makes the layout 4 / 1 heads
def test_golden_vote_example_through_ts_select():
    from golden_fixtures import vote_example
    ex = vote_example()
    n = ex["scores"].shape[1]
    offs = api.Offsets([0, n], dev())
    S = api.score_stride(offs)
    sc = np.zeros((4, S), np.float32)
    sc[:3, :n] = ex["scores"]
    scores = to_dev(sc)
    for sink, local, num, den, vmin, want in ex["selects"]:
        p = api.params(api.MODE_VOTE, (num, den), sink, local, vmin, (1, 2))
        sel = api.select(scores, offs, 1, p, want_theta=True, want_votes=True)
        torch.cuda.synchronize()
        assert np.array_equal(sel["idx"].cpu().numpy(), want)
        assert np.array_equal(f64(sel["theta"])[0], np.r_[ex["theta"], 0.0])
        assert np.array_equal(sel["votes"].cpu().numpy().astype(np.int32), ex["votes"])
    sink, local, num, den, _ = ex["perhead"][0]
    p = api.params(api.MODE_PER_HEAD, (num, den), sink, local, 1, (1, 2))
    sel = api.select(scores, offs, 1, p)
    torch.cuda.synchronize()
    K = sel["counts_host"][0]
    got = sel["idx"].cpu().numpy().reshape(4, K)
    for h, (_, _, _, _, want) in ex["perhead"].items():
        assert np.array_equal(got[h], want)
    assert np.array_equal(got[3], [0, 1, 2, 3, 10, 11])
