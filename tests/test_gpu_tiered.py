"""Decode over a tiered KV cache (ts_tiered_decode) and the batched index append from its ring.

TokenButler's inference layout keeps the newest N tokens in a circular buffer next to the rest of
the cache, appends the key projections N at a time, and can keep the rest of the cache in host
memory with only the selected rows read across the host link.  The tiered decode must equal the
oracle's decode on the logical cache (position t of sequence b from ring slot t mod N when
t >= n_b - N, else from the main store) within the 2e-3 bound of every decode test, and the GPU's
plain decode of the logical cache within 1e-5 (they differ only in how the split-K sums are
grouped).  Rows of the main store that the ring shadows, and ring slots that hold no position,
are filled with large values so that reading them would show.  With the main store in pinned
host memory the result must be bit-identical to the same call with the main store on the device.
The step loop at the end runs TokenButler's cadence: the index gets the ring's N rows at once
every N steps, the selection covers the indexed prefix, the selection expansion adds the current
sink and local window, and the tiered decode reads the ring for the newest tokens.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

from gpu_util import bits, dev, f64, to_dev

pytestmark = pytest.mark.gpu

POISON = int(synth.f32_to_bf16_bits(np.array([300.0], np.float32))[0])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def split_tiers(K, offsets, N):
    """The main store (shadowed rows poisoned) and the ring [B][N][Hkv][128] (unused slots
    poisoned) that hold the logical cache K."""
    B = len(offsets) - 1
    main = K.copy()
    ring = np.full((B, N) + K.shape[1:], POISON, np.uint16)
    for b in range(B):
        s, e = int(offsets[b]), int(offsets[b + 1])
        n = e - s
        for t in range(max(0, n - N), n):
            ring[b, t % N] = K[s + t]
            main[s + t] = POISON
    return main, ring


def random_lists(rng, offsets, frac, mode, Hq):
    """Ascending random lists in the ts_select layout (one per sequence, or one per head)."""
    lists, counts = [], []
    for b in range(len(offsets) - 1):
        n = int(offsets[b + 1] - offsets[b])
        k = max(1, int(n * frac))
        counts.append(k)
        for _ in range(1 if mode == api.MODE_VOTE else Hq):
            lists.append(np.sort(rng.choice(n, size=k, replace=False)).astype(np.int32))
    return np.concatenate(lists), counts


def run_both(x, N, mode, idx_np=None, counts=None, host=False):
    """Tiered decode of the logical cache x.K / x.V with a ring of N, and the plain decode."""
    offs = api.Offsets(x.offsets, dev())
    Km, Kr = split_tiers(x.K, x.offsets, N)
    Vm, Vr = split_tiers(x.V, x.offsets, N)
    q = to_dev(x.q)
    Kr_d, Vr_d = to_dev(Kr), to_dev(Vr)
    if host:
        Km_t = torch.from_numpy(Km.view(np.int16)).pin_memory()
        Vm_t = torch.from_numpy(Vm.view(np.int16)).pin_memory()
    else:
        Km_t, Vm_t = to_dev(Km), to_dev(Vm)
    if mode == api.MODE_DENSE:
        out = api.tiered_decode(q, Km_t, Vm_t, Kr_d, Vr_d, offs, mode)
        ref_gpu = api.dense_decode(q, to_dev(x.K), to_dev(x.V), offs)
    else:
        idx = to_dev(idx_np)
        cd = torch.tensor(counts, dtype=torch.int64, device=dev())
        out = api.tiered_decode(q, Km_t, Vm_t, Kr_d, Vr_d, offs, mode, idx, cd, counts)
        ref_gpu = api.sparse_decode(q, to_dev(x.K), to_dev(x.V), offs, idx, cd, counts, mode)
    torch.cuda.synchronize()
    return out, ref_gpu


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD, api.MODE_DENSE])
@pytest.mark.parametrize("lens,Hq,Hkv,N", [([5000, 300, 17], 32, 8, 256), ([9000], 8, 2, 64), ([700, 4100], 4, 4, 1),
                                           ([130, 3000], 16, 2, 512), ([2000], 8, 1, 2048)])
def test_tiered_matches_logical_cache(mode, lens, Hq, Hkv, N):
    x = synth.make_decode(2, lens, Hq, Hkv, 4, False)
    rng = np.random.default_rng(sum(lens) + N + 3 * mode)
    idx_np = counts = None
    if mode != api.MODE_DENSE:
        idx_np, counts = random_lists(rng, x.offsets, 0.2, mode, Hq)
    print(f"tiered lens={lens} Hq={Hq} Hkv={Hkv} N={N} mode={mode}", flush=True)
    out, ref_gpu = run_both(x, N, mode, idx_np, counts)
    if mode == api.MODE_DENSE:
        ref = O.dense_decode(x.q, x.K, x.V, x.offsets, Hq, Hkv)
    else:
        ref = O.decode(x.q, x.K, x.V, x.offsets, idx_np, np.array(counts), mode, Hq, Hkv)
    err = float(np.abs(f64(out) - ref).max())
    dif = float(np.abs(f64(out) - f64(ref_gpu)).max())
    print(f"  max abs error {err:.3g}, against the plain decode {dif:.3g}", flush=True)
    assert err <= 2e-3, f"tiered decode max abs error {err}"
    assert dif <= 1e-5, f"tiered decode differs from the plain decode by {dif}"


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_DENSE])
def test_tiered_host_offload(mode):
    """The main store in pinned host memory (the offloaded tier): the same bits as on the device."""
    x = synth.make_decode(2, [20000, 3000], 32, 8, 8, False)
    rng = np.random.default_rng(41)
    idx_np = counts = None
    if mode != api.MODE_DENSE:
        idx_np, counts = random_lists(rng, x.offsets, 0.2, mode, 32)
    print(f"host offload mode={mode}", flush=True)
    out_host, _ = run_both(x, 256, mode, idx_np, counts, host=True)
    out_dev, _ = run_both(x, 256, mode, idx_np, counts, host=False)
    assert torch.equal(out_host, out_dev), "offloaded main store changes the result"
    if mode == api.MODE_DENSE:
        ref = O.dense_decode(x.q, x.K, x.V, x.offsets, 32, 8)
    else:
        ref = O.decode(x.q, x.K, x.V, x.offsets, idx_np, np.array(counts), mode, 32, 8)
    assert float(np.abs(f64(out_host) - ref).max()) <= 2e-3


@pytest.mark.parametrize("mode", [api.MODE_VOTE, api.MODE_PER_HEAD])
def test_ring_cadence_steps(mode):
    """Decode steps with TokenButler's cadence on one 6000-token sequence, ring of 64 tokens,
    local window 256: each step writes the new token's K/V into ring slot t mod 64; when the
    length reaches a multiple of 64 the ring's 64 index rows are appended in one call and the ring
    is copied to the main store.  The selection covers the indexed prefix [0, m), the expansion
    (radius 0) adds the sink and the current local window, and the tiered decode reads the ring
    for the newest 64 positions.  Checked per step: the index rows equal the oracle's projection,
    the prefix selection equals the oracle's on the GPU's scores, the expanded list equals the
    oracle's expansion, and the decode is within 2e-3 of the oracle's decode of the whole cache."""
    N, Hq, Hkv = 64, 8, 2
    n0, steps = 6000 - 3, 2 * N + 6
    total = n0 + steps
    x = synth.make_decode(2, [total], Hq, Hkv, 8, False)
    P = to_dev(x.P)
    p = api.params(mode, (1, 5))
    vote = mode == api.MODE_VOTE
    # state before the first step: index rows and main store for [0, floor(n0 / N) N), the ring
    # holding [n0 - N, n0) at slot t mod N
    m0 = n0 // N * N
    kidx = torch.zeros((total, Hkv, 32), dtype=torch.int16, device=dev())
    api.index_append(to_dev(x.K[:m0]), P, kidx, 0)
    Km = torch.full((total, Hkv, 128), POISON, dtype=torch.int16, device=dev())
    Vm = torch.full((total, Hkv, 128), POISON, dtype=torch.int16, device=dev())
    Km[:m0] = to_dev(x.K[:m0])
    Vm[:m0] = to_dev(x.V[:m0])
    Kr = torch.zeros((1, N, Hkv, 128), dtype=torch.int16, device=dev())
    Vr = torch.zeros((1, N, Hkv, 128), dtype=torch.int16, device=dev())
    for t in range(n0 - N, n0):
        Kr[0, t % N] = to_dev(x.K[t])
        Vr[0, t % N] = to_dev(x.V[t])
    idx_ref_full = O.index_project(x.K, x.P)
    rng = np.random.default_rng(7 + mode)
    for step in range(steps):
        t_new = n0 + step
        n = t_new + 1
        Kr[0, t_new % N] = to_dev(x.K[t_new])
        Vr[0, t_new % N] = to_dev(x.V[t_new])
        if n % N == 0:
            # batched append of the ring's N index rows, then the ring moves to the main store
            api.index_append(Kr[0], P, kidx, n - N)
            Km[n - N:n] = Kr[0]
            Vm[n - N:n] = Vr[0]
        m = n // N * N
        q = synth.normal_bf16(rng, (1, Hq, 128))
        pre = api.Offsets(np.array([0, m], np.int64), dev())
        sel = api.score_select(to_dev(q), P, kidx, pre, Hkv, p, want_theta=vote, want_votes=vote)
        cur = api.Offsets(np.array([0, n], np.int64), dev())
        lists = 1 if vote else Hq
        exr = api.expand_selection(sel["idx"], sel["count"], sel["counts_host"], cur, lists=lists, radius=0)
        ex = exr["idx"]
        out = api.tiered_decode(to_dev(q), Km, Vm, Kr, Vr, cur, mode, ex, exr["caps"], exr["caps_host"])
        torch.cuda.synchronize()
        print(f"step {step}: n={n} indexed={m}", flush=True)
        assert np.array_equal(bits(kidx[:m]), idx_ref_full[:m]), "index rows differ from the oracle's projection"
        s64 = f64(sel["scores"])[:, :m]
        offm = np.array([0, m], np.int64)
        if vote:
            th = O.theta(s64, offm, 9, 10)
            v = O.votes(s64, th, offm)
            ref_sel, ref_cnt = O.select_vote(v, offm, 1, 5)
        else:
            ref_sel, ref_cnt = O.select_per_head(s64, offm, 1, 5)
        assert np.array_equal(sel["idx"].cpu().numpy(), ref_sel), "prefix selection differs from the oracle"
        ref_ex, _, ref_caps = O.expand_selection(ref_sel, ref_cnt, np.array([0, n], np.int64), lists=lists, radius=0)
        assert np.array_equal(ex.cpu().numpy(), ref_ex), "expanded list differs from the oracle"
        ref = O.decode(q, x.K[:n], x.V[:n], np.array([0, n], np.int64), ref_ex, np.array(ref_caps), mode, Hq, Hkv)
        err = float(np.abs(f64(out) - ref).max())
        assert err <= 2e-3, f"step {step}: decode max abs error {err}"
