"""ts_sparse_decode_noalloc against ts_sparse_decode through the C ABI.

Two calls in a row on one device, the second with a smaller input (another mode, fewer heads and
tokens): each output must equal ts_sparse_decode's on the same lists bit for bit (same kernels,
same launch shape) and the oracle's within the decode tolerance (max abs 2e-3).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

from gpu_util import Step, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def _one(x, mode):
    st = Step(x, mode=mode).run()
    sel = st.sel
    ref_out = st.out.clone()
    out = api.sparse_decode_noalloc(st.q, st.K, st.V, st.offs, sel["idx"], sel["count"], sel["counts_host"], mode)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "no-allocation decode differs from ts_sparse_decode"
    ref = O.decode(x.q, x.K, x.V, x.offsets, sel["idx"].cpu().numpy(), np.array(sel["counts_host"]), mode,
                   x.Hq, x.Hkv)
    err = float(np.abs(f64(out) - ref).max())
    assert err <= 2e-3, err
    return out, err


def test_noalloc_decode_two_calls():
    big = synth.make_decode(4, [30000, 9000], 32, 8, 64, False, (1, 5), 21)     # 7660 list entries
    small = synth.make_decode(1, [4096], 8, 2, 16, False, (1, 10), 22)          # 409 per head
    out1, e1 = _one(big, api.MODE_VOTE)
    keep = out1.clone()
    out2, e2 = _one(small, api.MODE_PER_HEAD)
    torch.cuda.synchronize()
    assert torch.equal(out1, keep), "a later call changed an earlier call's output"
    print("noalloc decode errors", e1, e2)
