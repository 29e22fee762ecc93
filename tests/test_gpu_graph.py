"""A decode step captured in a HIP graph replays to the eager step's results bit for bit.

The step is ts_score_select (with the append of the last token's index row) followed by
ts_sparse_decode, on buffers and workspaces the caller owns.  Between the replays an eager step
on another query runs on the same buffers and workspaces, so a replay that depended on what an
earlier call left in them would differ.  The kernels issue no memset nodes.
"""
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
def test_graph_replays_equal_eager(mode):
    x = synth.config2()
    Hq, Hkv = x.Hq, x.Hkv
    n = int(x.offsets[-1])
    q, K, V, P = to_dev(x.q), to_dev(x.K), to_dev(x.V), to_dev(x.P)
    q2 = torch.flip(q, dims=[1]).contiguous()          # another query: heads in reverse order
    offs = api.Offsets(x.offsets, dev())
    p = api.params(mode, x.budget)
    kidx = torch.empty((n, Hkv, 32), dtype=torch.int16, device=dev())
    api.index_append(K[:n - 1], P, kidx[:n - 1], 0)
    k_tot = api.budget_tokens(n, p)
    reps = Hq if mode == api.MODE_PER_HEAD else 1
    scores = torch.empty((Hq, api.score_stride(offs)), dtype=torch.float32, device=dev())
    idx = torch.empty(k_tot * reps, dtype=torch.int32, device=dev())
    count = torch.empty(1, dtype=torch.int64, device=dev())
    out = torch.empty((1, Hq, 128), dtype=torch.float32, device=dev())
    ws_s = torch.empty(api.score_select_workspace_bytes(offs, Hq, p), dtype=torch.uint8, device=dev())
    ws_d = torch.empty(api.decode_workspace_bytes(offs, [k_tot], Hq, Hkv, mode), dtype=torch.uint8, device=dev())

    def step(qq):
        sel = api.score_select(qq, P, kidx, offs, Hkv, p, K_last=K, ws=ws_s, scores=scores, idx=idx, count=count)
        api.sparse_decode(qq, K, V, offs, sel["idx"], sel["count"], sel["counts_host"], mode, ws=ws_d, out=out)

    def snapshot():
        torch.cuda.synchronize()
        return scores[:, :n].clone(), idx.clone(), count.clone(), out.clone()

    step(q)
    ref = snapshot()
    step(q2)
    ref2 = snapshot()
    assert not torch.equal(ref[1], ref2[1]), "the second query should select other tokens"

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(q)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(q)
    torch.cuda.synchronize()

    for r in range(4):
        step(q2)
        got2 = snapshot()
        for a, b in zip(got2, ref2):
            assert torch.equal(a, b), f"eager step between replays differs (round {r})"
        g.replay()
        got = snapshot()
        for name, a, b in zip(("scores", "idx", "count", "out"), got, ref):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager step"
    assert np.isfinite(ref[3].cpu().numpy()).all()
