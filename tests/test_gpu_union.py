"""Per-KV-group union of per-head lists (ts_union_lists) and the decode through it
(ts_union_decode) on the GPU.

The union, its head masks and sizes must equal the oracle's (a plain set union per group) bit for
bit on the same lists.  The union decode must match the oracle's per-head decode of the lists the
union was built from within max-abs 2e-3 (the tolerance of every decode test here), and the GPU
per-head decode of those lists within the same bound.  The lists are the oracle's own per-head
selections on its fp64 scores, or seeded random ascending lists whose heads share part of their
tokens (with -1 slots after the tokens, as in an expanded list).  Cases span several 4096-token
windows with a ragged tail, a one-token sequence, every head layout, identical, disjoint and full
lists, and the 128K-token layer of the LLaMA-3-8B shape at a 20 % budget.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

from gpu_util import dev, f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def random_lists(rng, lens, ks, Hq, Hkv, pad_frac=0.0):
    """Per-head lists in ts_select's layout: head h of sequence b takes k_b tokens, about half
    of them from a hot set shared by its KV group; with pad_frac > 0 a random share of each
    list's tail is -1 (an expanded list's empty slots)."""
    G = Hq // Hkv
    out = []
    for n, k in zip(lens, ks):
        for g in range(Hkv):
            hot = rng.choice(n, size=min(n, 2 * k), replace=False)
            for _ in range(G):
                a = rng.choice(hot, size=min(len(hot), k // 2), replace=False)
                rest = np.setdiff1d(np.arange(n), a, assume_unique=False)
                b = rng.choice(rest, size=k - len(a), replace=False)
                lst = np.sort(np.concatenate([a, b])).astype(np.int32)
                if pad_frac > 0 and k > 1:
                    v = int(rng.integers(int(k * (1 - pad_frac)), k + 1))
                    lst = np.concatenate([lst[:v], np.full(k - v, -1, np.int32)])
                out.append(lst)
    return np.concatenate(out).astype(np.int32)


def run_union(idx_np, lens, ks, Hq, Hkv):
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    offs = api.Offsets(offsets, dev())
    idx = to_dev(idx_np)
    cd = torch.tensor(ks, dtype=torch.int64, device=dev())
    uidx, umask, ucount = api.union_lists(idx, cd, ks, offs, Hq, Hkv)
    torch.cuda.synchronize()
    return offsets, offs, idx, cd, uidx, umask, ucount


def check_union(idx_np, lens, ks, Hq, Hkv):
    offsets, offs, idx, cd, uidx, umask, ucount = run_union(idx_np, lens, ks, Hq, Hkv)
    ru, rm, rc = O.union_lists(idx_np, np.array(ks), offsets, Hq, Hkv)
    assert np.array_equal(ucount.cpu().numpy(), rc), "union sizes differ from the oracle"
    assert np.array_equal(uidx.cpu().numpy(), ru), "union lists differ from the oracle"
    assert np.array_equal(umask.cpu().numpy(), rm), "head masks differ from the oracle"
    return offsets, offs, idx, cd, uidx, umask, ucount


@pytest.mark.parametrize("lens,frac,Hq,Hkv,pad", [
    ([4096 * 3 + 17, 1, 4096, 9000], 0.2, 8, 2, 0.0),
    ([20000], 0.2, 32, 8, 0.0),
    ([5000, 300], 0.3, 4, 4, 0.0),
    ([12289], 0.1, 8, 1, 0.0),
    ([4096 * 3 + 17, 700, 8192], 0.2, 16, 4, 0.3),
    ([4095, 4097], 0.5, 2, 1, 0.5),
])
def test_union_matches_oracle(lens, frac, Hq, Hkv, pad):
    rng = np.random.default_rng(sum(lens) + Hq)
    ks = [max(1, int(n * frac)) for n in lens]
    print(f"union lens={lens} ks={ks} Hq={Hq} Hkv={Hkv} pad={pad}", flush=True)
    check_union(random_lists(rng, lens, ks, Hq, Hkv, pad), lens, ks, Hq, Hkv)


def test_union_special_lists():
    """Identical lists: the list with every head bit; disjoint lists: all G k tokens with one bit
    each; full lists (k = n): every token with every bit; G = 1: the head's own list."""
    n, k, Hq = 10000, 2500, 4
    rng = np.random.default_rng(5)
    lst = np.sort(rng.choice(n, size=k, replace=False)).astype(np.int32)
    check_union(np.tile(lst, Hq), [n], [k], Hq, 1)
    dis = np.concatenate([np.arange(h, 4 * k, 4) for h in range(Hq)]).astype(np.int32)
    _, _, _, _, uidx, umask, ucount = check_union(dis, [n], [k], Hq, 1)
    assert int(ucount[0, 0]) == Hq * k and np.all(umask.cpu().numpy() == np.tile(1 << np.arange(Hq), k))
    full = np.tile(np.arange(n, dtype=np.int32), Hq)
    _, _, _, _, uidx, umask, ucount = check_union(full, [n], [n], Hq, 1)
    assert int(ucount[0, 0]) == n and np.all(umask.cpu().numpy()[:n] == 15)
    check_union(dis, [n], [k], Hq, Hq)


def _decode_both(x, idx_np, ks, offs_np):
    """GPU union + union decode and GPU per-head decode of the same lists, against the oracle."""
    Hq, Hkv = x.Hq, x.Hkv
    lens = [int(v) for v in np.diff(offs_np)]
    offsets, offs, idx, cd, uidx, umask, ucount = check_union(idx_np, lens, ks, Hq, Hkv)
    q, K, V = to_dev(x.q), to_dev(x.K), to_dev(x.V)
    out_u = api.union_decode(q, K, V, offs, uidx, umask, ucount, cd, ks)
    out_p = api.sparse_decode(q, K, V, offs, idx, cd, ks, api.MODE_PER_HEAD)
    torch.cuda.synchronize()
    ref = O.decode(x.q, x.K, x.V, offsets, idx_np, np.array(ks), api.MODE_PER_HEAD, Hq, Hkv)
    eu = float(np.abs(f64(out_u) - ref).max())
    ep = float(np.abs(f64(out_u) - f64(out_p)).max())
    print(f"union decode err {eu:.3g}, vs per-head decode {ep:.3g}", flush=True)
    assert eu <= 2e-3, f"union decode max abs error {eu}"
    assert ep <= 2e-3, f"union decode differs from the per-head decode by {ep}"


def test_union_decode_oracle_selection_c2():
    """The oracle's per-head 20 % selection of the 32K-token LLaMA-3-8B-shaped layer."""
    x = synth.config2()
    kidx = O.index_project(x.K, x.P)
    s = O.score(x.q, x.P, kidx, x.offsets, x.Hq, x.Hkv)
    bn, bd = x.budget
    idx_np, ks = O.select_per_head(s, x.offsets, bn, bd, 4, 256)
    _decode_both(x, idx_np, [int(k) for k in ks], x.offsets)


@pytest.mark.parametrize("lens,Hq,Hkv,pad", [([9000, 1, 4096 * 2 + 5], 8, 2, 0.0), ([5000, 12000], 32, 8, 0.3),
                                           ([3000], 4, 4, 0.2), ([6000], 8, 1, 0.0)])
def test_union_decode_ragged(lens, Hq, Hkv, pad):
    x = synth.make_decode(1, lens, Hq, Hkv, 8, False)
    rng = np.random.default_rng(len(lens) * 100 + Hq)
    ks = [max(1, n // 5) for n in lens]
    print(f"union decode lens={lens} Hq={Hq} Hkv={Hkv} pad={pad}", flush=True)
    _decode_both(x, random_lists(rng, lens, ks, Hq, Hkv, pad), ks, x.offsets)


def test_union_c3_full_size():
    """The 128K-token layer (32 query / 8 KV heads) at a 20 % budget: the oracle's per-head
    selection, its union on the GPU bit-exact, the union decode against the oracle's decode."""
    x = synth.config3(20)
    kidx = O.index_project(x.K, x.P)
    s = O.score(x.q, x.P, kidx, x.offsets, x.Hq, x.Hkv)
    bn, bd = x.budget
    idx_np, ks = O.select_per_head(s, x.offsets, bn, bd, 4, 256)
    del s
    print(f"c3 union: k={int(ks[0])}", flush=True)
    _decode_both(x, idx_np, [int(k) for k in ks], x.offsets)
