"""GPU parity of the fused score-and-select call (ts_score_select).

Its outputs must equal, bit for bit, those of ts_index_append + ts_score + ts_select on the
same inputs (the same index rows, score arithmetic and exact order statistics), and they are
checked stage by stage against the fp64 oracle with the rules of test_gpu_parity.  The cases
cover the bracket path (rows longer than the sample threshold), rows short enough to take
every key as a candidate, the whole-row fallback (heavy ties, rows whose bracket holds more
keys than the LDS capacity), ragged batches, every head layout and the full-size workloads.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

from gpu_util import FusedStep, Step, assert_same_step, check_staged, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def both(x, **kw):
    a = Step(x, **kw).run()
    b = FusedStep(x, **kw).run()
    assert_same_step(a, b)
    return b


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_c1_c2(mode):
    print("c1", check_staged(both(synth.config1(), mode=mode)))
    print("c2", check_staged(both(synth.config2(), mode=mode)))


@pytest.mark.parametrize("lengths,budget", [([5000, 1234, 300, 4097], (3, 20)), ([70000, 20000], (1, 5)),
                                            ([1, 64, 65, 20000], (1, 10))])
@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_ragged(lengths, budget, mode):
    x = synth.make_decode(4, lengths, 32, 8, lambda n: n // 100, False, budget, 3)
    check_staged(both(x, mode=mode))


# more sequences than the 64 lanes of a wave: every kernel's sequence lookup takes two or
# three rounds (lane i % 64 loads sequence i), with lengths from 1 token (shorter than sink +
# local) to several 64-token tiles mixed in one batch
@pytest.mark.parametrize("B", [70, 130])
@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_many_sequences(B, mode):
    lengths = np.random.default_rng(B).integers(1, 700, size=B)
    x = synth.make_decode(4, lengths, 8, 2, lambda n: n // 100, False, (1, 5), 13)
    st = both(x, mode=mode, local=64)
    check_staged(st)
    if mode == api.MODE_VOTE:
        dense = api.dense_decode(st.q, st.K, st.V, st.offs)
        torch.cuda.synchronize()
        assert np.abs(f64(dense) - O.dense_decode(x.q, x.K, x.V, x.offsets, 8, 2)).max() <= 2e-3


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (2, 1), (4, 1), (8, 1), (2, 2), (4, 2), (8, 2), (16, 2), (4, 4), (8, 4),
                                    (16, 4), (32, 4), (8, 8), (16, 8), (32, 8), (64, 8)])
@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_head_layouts(Hq, Hkv, mode):
    x = synth.make_decode(4, [20000, 700], Hq, Hkv, 8, False, (1, 5), 11)
    both(x, mode=mode, local=64)


def test_short_and_special():
    for n in (1, 5, 259, 260, 261):
        x = synth.make_decode(1, [n], 8, 2, 0, False, (1, 10), n)
        check_staged(both(x))
    x = synth.make_decode(1, [5000], 8, 2, 0, False, (1, 10), 2)
    x.q[:] = 0
    for mode in (api.MODE_VOTE, api.MODE_PER_HEAD):
        st = both(x, mode=mode)
        assert np.all(f64(st.scores)[:, :5000] == 0)
        assert np.array_equal(st.sel["idx"].cpu().numpy()[:500], np.r_[0:244, 4744:5000])
    x = synth.config1()
    check_staged(both(x, theta=(1, 2)))
    check_staged(both(x, vmin=3))
    check_staged(both(x, sink=0, local=0))
    x = synth.make_decode(1, [3000], 8, 2, 16, False, (1, 1), 5)
    st = both(x)
    assert np.array_equal(st.sel["idx"].cpu().numpy(), np.arange(3000))


# thresholds inside a mass of tied scores (the sampled bracket collapses onto the tied key, or
# the target rank falls outside it) and a row whose bracket holds more keys than fit in LDS:
# both go through the whole-row radix select
@pytest.mark.parametrize("zero_frac", [1.0, 0.95])
def test_heavy_ties(zero_frac):
    x = synth.make_decode(1, [40000], 8, 2, 0, False, (1, 5), 6)
    rows = np.random.default_rng(6).permutation(40000)[:int(40000 * zero_frac)]
    x.K[rows] = 0
    for mode in (api.MODE_VOTE, api.MODE_PER_HEAD):
        check_staged(both(x, mode=mode))


# rows of few distinct keys: the bracket around the threshold holds whole runs of tied keys, so
# tiles hold more in-bracket keys than their slots (the overflow keys go through LDS, or through
# memory when more than fit), and the answer's digit holds hundreds of keys (radix select in LDS)
@pytest.mark.parametrize("n, distinct", [(40000, 12), (40000, 150), (40000, 2000), (80000, 3)])
def test_bracket_paths(n, distinct):
    x = synth.make_decode(1, [n], 8, 2, 0, False, (1, 5), 8)
    rng = np.random.default_rng(distinct)
    base = x.K[rng.permutation(n)[:distinct]]
    x.K = np.ascontiguousarray(base[rng.integers(0, distinct, n)])
    for mode in (api.MODE_VOTE, api.MODE_PER_HEAD):
        check_staged(both(x, mode=mode))


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_long_row(mode):
    x = synth.make_decode(3, [300000], 8, 2, 300, False, (1, 5), 9)
    check_staged(both(x, mode=mode))


# the benchmarked workload at full size: LLaMA-3-8B-shaped layer, n = 131072 + 1 (the step's
# appended token), 20 % budget, both modes; the decode of the GPU lists is checked in full
@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_c3_full_size(mode):
    x = synth.config3(20, 131072)
    q1, k1, v1 = synth.config3_step(1, x.q, x.Hkv)
    x.K = np.concatenate([x.K, k1])
    x.V = np.concatenate([x.V, v1])
    x.q = q1
    x.offsets = np.array([0, 131073], np.int64)
    r = check_staged(both(x, mode=mode))
    print("c3 full", mode, r)


# the ragged Mistral-7B-shaped batch at full size (16 sequences of 16K-64K tokens, 15 %)
def test_c4_full_size():
    x = synth.config4()
    r = check_staged(both(x))
    print("c4 full", r)
