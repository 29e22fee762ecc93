"""Selection reuse with neighbour fetch on the GPU (ts_expand_selection) and the sparse decode of
the expanded lists, whose empty slots (-1) it skips.

Expanded lists must equal the oracle's expansion of the GPU's own earlier lists bit for bit; the
decode of an expanded list must match the oracle's decode of that list within max-abs 2e-3 (the
oracle skips the empty slots too).  Cases: the vote list of the LLaMA-3-8B-shaped layer at 32K
tokens and the per-head lists of the tiny layer (radius 0, 1, 2), a ragged batch, a sequence that
grew by a few decode steps since its selection (its local window moves), and lists whose
sequences are shorter than sink + local.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

from gpu_util import Step, dev, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def _expand_and_check(q, K, V, x_now, offs_now, sel_idx, counts_prev, mode, Hq, Hkv, radius, sink=4, local=256):
    lists = Hq if mode == api.MODE_PER_HEAD else 1
    cp = torch.tensor(counts_prev, dtype=torch.int64, device=dev())
    ex = api.expand_selection(sel_idx, cp, counts_prev, offs_now, lists, sink, local, radius)
    out = api.sparse_decode(q, K, V, offs_now, ex["idx"], ex["caps"], ex["caps_host"], mode)
    torch.cuda.synchronize()
    ref, cnt, caps = O.expand_selection(sel_idx.cpu().numpy(), counts_prev, x_now.offsets, lists, sink, local, radius)
    got = ex["idx"].cpu().numpy()
    assert caps == ex["caps_host"] and np.array_equal(ex["caps"].cpu().numpy(), caps)
    assert np.array_equal(got, ref), "expanded lists differ from the oracle"
    assert np.array_equal(ex["valid"].cpu().numpy(), cnt)
    want = O.decode(x_now.q, x_now.K, x_now.V, x_now.offsets, got, np.array(caps), mode, Hq, Hkv)
    err = float(np.abs(f64(out) - want).max())
    assert err <= 2e-3, err
    return {"valid": int(cnt.sum()), "capacity": int(sum(caps)) * lists, "decode_err": err}


@pytest.mark.parametrize("radius", [0, 1, 2])
def test_expand_vote_c2(radius):
    st = Step(synth.config2()).run()
    r = _expand_and_check(st.q, st.K, st.V, st.x, st.offs, st.sel["idx"], st.sel["counts_host"], api.MODE_VOTE,
                          st.Hq, st.Hkv, radius)
    print("c2 vote radius", radius, r)


@pytest.mark.parametrize("radius", [0, 1, 2])
def test_expand_per_head_c1(radius):
    st = Step(synth.config1(), mode=api.MODE_PER_HEAD).run()
    r = _expand_and_check(st.q, st.K, st.V, st.x, st.offs, st.sel["idx"], st.sel["counts_host"],
                          api.MODE_PER_HEAD, st.Hq, st.Hkv, radius)
    print("c1 per-head radius", radius, r)


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_expand_ragged_and_short(mode):
    # sequences shorter than sink + local (everything is kept) next to longer ones
    x = synth.make_decode(4, [5000, 100, 257, 9000], 32, 8, lambda n: n // 100, False, (3, 20), 3)
    st = Step(x, mode=mode).run()
    r = _expand_and_check(st.q, st.K, st.V, st.x, st.offs, st.sel["idx"], st.sel["counts_host"], mode, st.Hq,
                          st.Hkv, 1)
    print("ragged", mode, r)


def test_reuse_after_steps():
    """A selection made at n0 tokens, reused after the sequence grew by 1, 2 and 5 decode steps:
    the current local window moves with n, the earlier selection keeps its positions."""
    n0, grow = 20000, 5
    full = synth.make_decode(6, [n0 + grow], 32, 8, 200, True, (1, 5), 0)
    prefix = synth.DecodeInputs(6, 32, 8, np.array([0, n0], np.int64), full.q, full.K[:n0], full.V[:n0], full.P,
                                (1, 5))
    st = Step(prefix).run()
    for g in (1, 2, grow):
        x_now = synth.DecodeInputs(6, 32, 8, np.array([0, n0 + g], np.int64), full.q, full.K[:n0 + g],
                                   full.V[:n0 + g], full.P, (1, 5))
        offs_now = api.Offsets(x_now.offsets, dev())
        K, V = to_dev(x_now.K), to_dev(x_now.V)
        r = _expand_and_check(st.q, K, V, x_now, offs_now, st.sel["idx"], st.sel["counts_host"], api.MODE_VOTE,
                              32, 8, 1)
        print("reuse after", g, "steps", r)


def test_expand_empty_previous_list():
    """A previous list with no entries keeps only the current forced tokens (no entry is read)."""
    x = synth.make_decode(8, [3000, 2000], 8, 2, 4, False, (1, 5), 0)
    offs = api.Offsets(x.offsets, dev())
    prev = torch.zeros(4, dtype=torch.int32, device=dev())
    cp = torch.zeros(2, dtype=torch.int64, device=dev())
    ex = api.expand_selection(prev, cp, [0, 0], offs, 1, 4, 256, 2)
    torch.cuda.synchronize()
    ref, cnt, caps = O.expand_selection(np.zeros(0, np.int32), [0, 0], x.offsets, 1, 4, 256, 2)
    assert np.array_equal(ex["idx"].cpu().numpy(), ref) and np.array_equal(ex["valid"].cpu().numpy(), cnt)
