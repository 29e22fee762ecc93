"""GPU parity of snapkv_compress against the fp64 CPU oracle.

importance: |gpu - oracle| <= a per-element bound derived from the GPU arithmetic
  (gpu_util.snap_importance_bound: fp32 MFMA sums of exact bf16 products, the log2-domain
  scaling, exp2, the softmax-denominator and column-sum chains); the observed maximum error
  relative to the bound is printed;
pooled: within 4 ulp-level relative error of the oracle's pooling of the GPU importance;
indices: bit-exact against the oracle's top-c of the GPU pooled values;
K/V: bit copies of the selected rows.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

from gpu_util import bits, check_snap_endtoend, f64, snap_importance_bound, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def _run(x):
    r = api.snapkv_compress(to_dev(x.q_obs), to_dev(x.K), to_dev(x.V), x.c, 3, want_importance=True)
    torch.cuda.synchronize()
    return r


def _check_selection(x, r):
    pooled = f64(r["pooled"])
    imp = f64(r["importance"])
    ref_pool = O.avg_pool1d(imp, 3)
    assert np.all(np.abs(pooled - ref_pool) <= 4 * 2.0 ** -24 * np.abs(ref_pool) + 1e-30)
    idx = r["idx"].cpu().numpy()
    assert np.array_equal(idx, O.topc(pooled, x.c)), "top-c differs from the oracle on the GPU pooled values"
    Ko, Vo = O.gather_rows(x.K, x.V, idx)
    assert np.array_equal(bits(r["K"]), Ko) and np.array_equal(bits(r["V"]), Vo)
    return idx


def _check_importance(x, r, groups=None):
    """GPU importance within the derived per-element bound of the oracle's (the loop oracle
    for small n, its matmul form, pinned against it, at full size).  Returns the observed
    maximum of error / bound and of the relative error."""
    imp = f64(r["importance"])
    Hq, Hkv = x.Hq, x.Hkv
    groups = list(range(Hkv)) if groups is None else groups
    _, eb = snap_importance_bound(x.q_obs, x.K, Hq, Hkv, groups)
    if x.K.shape[0] <= 20000:
        full = O.snapkv_importance(x.q_obs, x.K, Hq, Hkv)
        ref = {g: full[g] for g in groups}
    else:
        ref = O.snapkv_importance_matmul(x.q_obs, x.K, Hq, Hkv, groups=groups)
    worst_b, worst_r = 0.0, 0.0
    for g in groups:
        err = np.abs(imp[g] - ref[g])
        assert np.all(err <= eb[g]), f"group {g}: error above the bound at {np.flatnonzero(err > eb[g])[:5]}"
        worst_b = max(worst_b, float(np.max(err / eb[g])))
        worst_r = max(worst_r, float(np.max(err / ref[g])))
    assert np.allclose(imp.sum(axis=1), 1.0, atol=1e-4)
    return {"max_err_over_bound": worst_b, "max_rel_err": worst_r}


@pytest.mark.parametrize("n,w,Hq,Hkv,c", [(3000, 8, 8, 2, 300), (777, 16, 4, 4, 100), (4096, 32, 64, 8, 512),
                                          (500, 4, 32, 8, 4096)])
def test_snapkv_small(n, w, Hq, Hkv, c):
    x = synth.make_snap(11, n, w, Hq, Hkv, max(1, n // 64), c)
    r = _run(x)
    stats = _check_importance(x, r)
    idx = _check_selection(x, r)
    if c >= n:
        assert np.array_equal(idx, np.tile(np.arange(n), (Hkv, 1)))
    stats.update(check_snap_endtoend(x, r))
    print("snapkv", n, w, Hq, Hkv, c, stats)


# row-tile counts R / 16 other than 1, 2 and 16 (each is its own kernel instantiation), on a
# sequence whose last key block and last 16-key tile are partial
@pytest.mark.parametrize("w,Hq,Hkv", [(12, 16, 4), (10, 64, 8), (24, 32, 8), (14, 64, 8), (22, 64, 8), (24, 64, 8),
                                      (26, 64, 8), (30, 64, 8)])
def test_snapkv_row_tiles(w, Hq, Hkv):
    x = synth.make_snap(12, 1500, w, Hq, Hkv, 20, 200)
    r = _run(x)
    stats = _check_importance(x, r)
    _check_selection(x, r)
    print("snapkv row tiles", w, Hq, Hkv, stats)


def test_snapkv_full_size_c5():
    x = synth.config5()
    r = _run(x)
    stats = _check_importance(x, r, groups=[0, 5])
    _check_selection(x, r)
    stats.update(check_snap_endtoend(x, r, groups=[0, 5]))
    print("snapkv c5", stats)


@pytest.mark.parametrize("k_cluster", [0, 1, 2])
def test_snapkv_cluster_retention(k_cluster):
    """Cluster-based retention of the GPU's top-c lists: widened lists, padding and the gathered
    rows bit-exact against the oracle on the same lists."""
    x = synth.make_snap(14, 5000, 8, 16, 4, 60, 400)
    r = _run(x)
    K, V = to_dev(x.K), to_dev(x.V)
    c = api.snapkv_retain_clusters(r["idx"], K, V, k_cluster)
    torch.cuda.synchronize()
    io, Ko, Vo, valid = O.snapkv_retain_clusters(x.K, x.V, r["idx"].cpu().numpy(), k_cluster)
    assert np.array_equal(c["idx"].cpu().numpy(), io)
    assert np.array_equal(c["valid"].cpu().numpy(), valid)
    assert np.array_equal(bits(c["K"]), Ko) and np.array_equal(bits(c["V"]), Vo)
    print("cluster", k_cluster, "kept", valid.tolist(), "of capacity", io.shape[1])
