"""GPU parity of snapkv_compress against the fp64 CPU oracle.

importance: |gpu - oracle| <= 3e-4 * oracle + 1e-10 (fp32 MFMA scores: the 128-term
  bf16 products are exact and the fp32 sum error is below 128 u sum|q k| / sqrt(128); the
  exp2 of an fp32 argument adds a few ulp; the bound covers |s| up to ~25);
pooled: within 4 ulp-level relative error of the oracle's pooling of the GPU importance;
indices: bit-exact against the oracle's top-c of the GPU pooled values;
K/V: bit copies of the selected rows.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

from gpu_util import bits, f64, to_dev

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


@pytest.mark.parametrize("n,w,Hq,Hkv,c", [(3000, 8, 8, 2, 300), (777, 16, 4, 4, 100), (4096, 32, 64, 8, 512),
                                          (500, 4, 32, 8, 4096)])
def test_snapkv_small(n, w, Hq, Hkv, c):
    x = synth.make_snap(11, n, w, Hq, Hkv, max(1, n // 64), c)
    r = _run(x)
    imp = f64(r["importance"])
    ref = O.snapkv_importance(x.q_obs, x.K, Hq, Hkv)
    err = np.abs(imp - ref)
    assert np.all(err <= 3e-4 * ref + 1e-10), f"importance error max rel {np.max(err / (ref + 1e-30))}"
    assert np.allclose(imp.sum(axis=1), 1.0, atol=1e-4)
    idx = _check_selection(x, r)
    if c >= n:
        assert np.array_equal(idx, np.tile(np.arange(n), (Hkv, 1)))
    print("rel err", float(np.max(err / ref)))


# row-tile counts R / 16 other than 1, 2 and 16 (each is its own kernel instantiation), on a
# sequence whose last key block and last 16-key tile are partial
@pytest.mark.parametrize("w,Hq,Hkv", [(12, 16, 4), (10, 64, 8), (24, 32, 8), (14, 64, 8), (22, 64, 8), (24, 64, 8),
                                      (26, 64, 8), (30, 64, 8)])
def test_snapkv_row_tiles(w, Hq, Hkv):
    x = synth.make_snap(12, 1500, w, Hq, Hkv, 20, 200)
    r = _run(x)
    imp = f64(r["importance"])
    ref = O.snapkv_importance(x.q_obs, x.K, Hq, Hkv)
    err = np.abs(imp - ref)
    assert np.all(err <= 3e-4 * ref + 1e-10), f"importance error max rel {np.max(err / (ref + 1e-30))}"
    _check_selection(x, r)


def test_snapkv_full_size_c5():
    x = synth.config5()
    r = _run(x)
    imp = f64(r["importance"])
    assert np.allclose(imp.sum(axis=1), 1.0, atol=1e-4)
    ref = O.snapkv_importance_matmul(x.q_obs, x.K, 64, 8, groups=[0, 5])
    for g, rg in ref.items():
        err = np.abs(imp[g] - rg)
        assert np.all(err <= 3e-4 * rg + 1e-10), f"group {g}: max rel {np.max(err / (rg + 1e-30))}"
    _check_selection(x, r)
