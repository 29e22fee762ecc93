"""Helpers for the GPU parity tests: device transfer, one staged decode step, bounds."""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

U = 2.0 ** -24   # fp32 unit roundoff


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def f64(t) -> np.ndarray:
    return t.cpu().numpy().astype(np.float64)


def score_bound(q, P, kidx, offsets, Hq, Hkv):
    """fp32 error bound of the index score, |gpu - exact| <= bound[h][t] (standard dot
    product bounds: gamma_n = n u for the 128-term projection, the scale and the 32-term
    dot product)."""
    qf = synth.bf16_bits_to_f32(q.reshape(-1)).reshape(q.shape).astype(np.float64)
    kf = synth.bf16_bits_to_f32(kidx.reshape(-1)).reshape(kidx.shape).astype(np.float64)
    Pa = np.abs(P.astype(np.float64))
    G = Hq // Hkv
    B = len(offsets) - 1
    out = np.zeros((Hq, int(offsets[-1])))
    for b in range(B):
        qp_abs = np.abs(qf[b]) @ Pa                  # [Hq][32]  sum_j |q_j P_jc|
        qp = qf[b] @ P.astype(np.float64)            # exact q'
        for h in range(Hq):
            ks = kf[offsets[b]:offsets[b + 1], h // G, :]
            err_q = (130 * U) * qp_abs[h]            # error of q'_c incl. the scale
            out[h, offsets[b]:offsets[b + 1]] = (np.abs(ks) @ err_q + 34 * U * (np.abs(ks) @ np.abs(qp[h]))) / np.sqrt(32)
    return out


class Step:
    """Runs the four step calls on the GPU and keeps every stage's output."""

    def __init__(self, x: synth.DecodeInputs, mode=api.MODE_VOTE, budget=None, theta=(9, 10), vmin=1,
                 sink=4, local=256):
        self.x = x
        self.Hq, self.Hkv = x.Hq, x.Hkv
        self.n = int(x.offsets[-1])
        self.q, self.K, self.V = to_dev(x.q), to_dev(x.K), to_dev(x.V)
        self.P = to_dev(x.P)
        self.offs = api.Offsets(x.offsets, dev())
        self.p = api.params(mode, budget or x.budget, sink, local, vmin, theta)
        self.mode = mode

    def run(self):
        x = self.x
        kidx = torch.empty((self.n, self.Hkv, 32), dtype=torch.int16, device=dev())
        api.index_append(self.K, self.P, kidx, 0)
        self.kidx = kidx
        self.scores = api.score(self.q, self.P, kidx, self.offs, self.Hkv)
        self.sel = api.select(self.scores, self.offs, self.Hkv, self.p, want_theta=True, want_votes=True)
        self.out = api.sparse_decode(self.q, self.K, self.V, self.offs, self.sel["idx"], self.sel["count"],
                                     self.sel["counts_host"], self.mode)
        torch.cuda.synchronize()
        return self


def check_staged(st: Step, decode_tol=2e-3):
    """Stage-by-stage parity of one GPU step against the oracle (see the module doc of
    test_gpu_parity for the rules)."""
    x = st.x
    offs = x.offsets
    p = st.p
    kidx = bits(st.kidx)
    assert np.array_equal(kidx, O.index_project(x.K, x.P)), "K_index differs from the oracle"
    sc = f64(st.scores)[:, :int(offs[-1])]
    ref = O.score(x.q, x.P, kidx, offs, st.Hq, st.Hkv)
    bound = score_bound(x.q, x.P, kidx, offs, st.Hq, st.Hkv)
    viol = np.abs(sc - ref) > 2 * bound + 1e-30
    assert not viol.any(), f"score outside bound at {np.argwhere(viol)[:5]}"
    counts = np.array(st.sel["counts_host"], np.int64)
    assert np.array_equal(st.sel["count"].cpu().numpy(), counts)
    idx = st.sel["idx"].cpu().numpy()
    if st.mode == api.MODE_VOTE:
        th_ref = O.theta(sc, offs, p.theta_num, p.theta_den)
        th = f64(st.sel["theta"])
        assert np.array_equal(th, th_ref), "theta is not the order statistic of the GPU scores"
        v_ref = O.votes(sc, th_ref, offs)
        v = st.sel["votes"].cpu().numpy().astype(np.int32)
        assert np.array_equal(v, v_ref), "votes differ from the oracle on the GPU scores"
        idx_ref, _ = O.select_vote(v, offs, p.budget_num, p.budget_den, p.sink, p.local, p.v_min)
        assert np.array_equal(idx, idx_ref), "vote selection differs from the oracle on the GPU votes"
    else:
        idx_ref, _ = O.select_per_head(sc, offs, p.budget_num, p.budget_den, p.sink, p.local)
        assert np.array_equal(idx, idx_ref), "per-head selection differs from the oracle on the GPU scores"
    out_ref = O.decode(x.q, x.K, x.V, offs, idx, counts, st.mode, st.Hq, st.Hkv)
    err = float(np.abs(f64(st.out) - out_ref).max())
    assert err <= decode_tol, f"decode max abs error {err}"
    return {"decode_err": err, "score_err": float(np.abs(sc - ref).max())}


class FusedStep(Step):
    """The same step through ts_score_select: the index of every sequence's last token is
    appended by the call itself (K_last), the rest of the index is built beforehand."""

    def run(self):
        kidx = torch.empty((self.n, self.Hkv, 32), dtype=torch.int16, device=dev())
        offs = self.x.offsets
        for b in range(len(offs) - 1):
            a, e = int(offs[b]), int(offs[b + 1])
            if e - 1 > a:
                api.index_append(self.K[a:e - 1], self.P, kidx[a:e - 1], 0)
        self.kidx = kidx
        self.sel = api.score_select(self.q, self.P, kidx, self.offs, self.Hkv, self.p, K_last=self.K,
                                    want_theta=True, want_votes=True)
        self.scores = self.sel["scores"]
        self.out = api.sparse_decode(self.q, self.K, self.V, self.offs, self.sel["idx"], self.sel["count"],
                                     self.sel["counts_host"], self.mode)
        torch.cuda.synchronize()
        return self


def assert_same_step(a: Step, b: Step):
    """Two runs of a step agree bit for bit: index, scores, thresholds, votes, lists, output."""
    n = a.n
    assert torch.equal(a.kidx, b.kidx), "index differs"
    assert torch.equal(a.scores[:, :n], b.scores[:, :n]), "scores differ"
    assert torch.equal(a.sel["count"], b.sel["count"])
    assert torch.equal(a.sel["idx"], b.sel["idx"]), "lists differ"
    if a.mode == api.MODE_VOTE:
        assert torch.equal(a.sel["theta"], b.sel["theta"]), "thresholds differ"
        assert torch.equal(a.sel["votes"], b.sel["votes"]), "votes differ"
    assert torch.equal(a.out, b.out), "decode output differs"
