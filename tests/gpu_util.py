"""Helpers for the GPU parity tests: device transfer, one staged decode step, bounds."""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle as O
from query_aware_sparse_index_amd import api, synth

U = 2.0 ** -24   # fp32 unit roundoff
D = 128


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


def check_staged(st: Step, decode_tol=2e-3, index_ref=None):
    """Stage-by-stage parity of one GPU step against the oracle (see the module doc of
    test_gpu_parity for the rules).  index_ref: the oracle's index rows when already computed."""
    x = st.x
    offs = x.offsets
    p = st.p
    kidx = bits(st.kidx)
    if index_ref is None:
        index_ref = O.index_project(x.K, x.P)
    assert np.array_equal(kidx, index_ref), "K_index differs from the oracle"
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


# ------------------------------------------------------------------ end to end
REL = 1e-5   # swaps are allowed only between keys within this relative distance of the boundary


def _boundary_diff(sel_gpu, sel_ref, key_ref, forced, tol):
    """Tokens in the symmetric difference of two equally sized selections; each must sit at
    the reference boundary key, i.e. |key_ref[t] - kappa| <= tol[t] with kappa the smallest
    reference key among the reference's selected non-forced tokens.  Returns (#diff, worst
    relative distance of a differing token from the boundary)."""
    a, r = set(int(t) for t in sel_gpu), set(int(t) for t in sel_ref)
    assert len(a) == len(sel_gpu) and len(r) == len(sel_ref) and len(a) == len(r)
    diff = sorted(a ^ r)
    if not diff:
        return 0, 0.0
    assert not any(forced(t) for t in diff), "a forced token is missing from one of the lists"
    nf = [t for t in r if not forced(t)]
    kappa = min(key_ref[t] for t in nf)
    worst = 0.0
    for t in diff:
        d = abs(key_ref[t] - kappa)
        assert d <= tol[t], f"token {t}: key {key_ref[t]} is {d} from the boundary {kappa} (tolerance {tol[t]})"
        worst = max(worst, d / max(abs(kappa), 1e-300))
    return len(diff), worst


def check_endtoend(st: Step):
    """End-to-end selection parity: the GPU lists against the oracle run end to end on its own
    fp64 scores (from the same index rows, which the staged check shows to be bit-exact); lists
    may differ only in tokens whose scores lie within 1e-5 relative of the selection boundary.
    Vote mode: every GPU vote is within #near(t) of the oracle's, where a head is near at t when
    |S_h(t) - theta_h| <= 1e-5 |theta_h| (+ the fp32 score bound as a floor), and every token in
    which the lists differ is a near token or carries the oracle's boundary key.
    Per-head mode: every token in which a head's lists differ has an oracle score within 1e-5
    relative (+ the bound floor) of that head's oracle boundary score."""
    x, p = st.x, st.p
    offs = x.offsets
    B, Hq, Hkv = len(offs) - 1, st.Hq, st.Hkv
    ntot = int(offs[-1])
    kidx = bits(st.kidx)
    s_o = O.score(x.q, x.P, kidx, offs, Hq, Hkv)
    bnd = score_bound(x.q, x.P, kidx, offs, Hq, Hkv)
    idx = st.sel["idx"].cpu().numpy()
    ks = [int(k) for k in st.sel["counts_host"]]
    ndiff, worst, nnear = 0, 0.0, 0
    if p.mode == api.MODE_VOTE:
        th_o = O.theta(s_o, offs, p.theta_num, p.theta_den)
        v_o = O.votes(s_o, th_o, offs)
        idx_o, _ = O.select_vote(v_o, offs, p.budget_num, p.budget_den, p.sink, p.local, p.v_min)
        v_g = st.sel["votes"].cpu().numpy().astype(np.int64)
        near = np.zeros(ntot, np.int64)
        for b in range(B):
            a, e = int(offs[b]), int(offs[b + 1])
            for h in range(Hq):
                tol = REL * abs(th_o[b, h]) + 2 * bnd[h, a:e] + 2 * bnd[h, a:e].max()
                near[a:e] += np.abs(s_o[h, a:e] - th_o[b, h]) <= tol
        nnear = int((near > 0).sum())
        bad = np.abs(v_g - v_o) > near
        assert not bad.any(), f"votes differ beyond the near ties at {np.flatnonzero(bad)[:5]}"
        kpre = 0
        for b in range(B):
            a, n, k = int(offs[b]), int(offs[b + 1] - offs[b]), ks[b]
            key = np.where(v_o[a:a + n] >= p.v_min, v_o[a:a + n], -1).astype(np.float64)
            tol = np.where(near[a:a + n] > 0, np.inf, 0.0)
            forced = lambda t: t < p.sink or t >= n - p.local
            d, w = _boundary_diff(idx[kpre:kpre + k], idx_o[kpre:kpre + k], key, forced, tol)
            ndiff += d
            kpre += k
    else:
        idx_o, _ = O.select_per_head(s_o, offs, p.budget_num, p.budget_den, p.sink, p.local)
        kpre = 0
        for b in range(B):
            a, n, k = int(offs[b]), int(offs[b + 1] - offs[b]), ks[b]
            forced = lambda t: t < p.sink or t >= n - p.local
            for h in range(Hq):
                lo = Hq * kpre + h * k
                key = s_o[h, a:a + n]
                sel_o = idx_o[lo:lo + k]
                nf = [t for t in sel_o if not forced(t)]
                kap = min(key[t] for t in nf) if nf else 0.0
                tb = bnd[h, a:a + n]
                tol = REL * np.maximum(np.abs(key), abs(kap)) + 2 * tb + 2 * tb.max()
                d, w = _boundary_diff(idx[lo:lo + k], sel_o, key, forced, tol)
                ndiff += d
                worst = max(worst, w)
            kpre += k
    return {"diff_tokens": ndiff, "near_tokens": nnear, "worst_rel_from_boundary": worst}


# ------------------------------------------------------------ SnapKV error bound
LOG2E = 1.4426950408889634


def snap_importance_bound(q_obs, K, Hq, Hkv, groups, chunk=8192):
    """Per-element bound of |gpu - exact| for the SnapKV importance, from the GPU arithmetic:
    scores s_rj = fp32 MFMA sums of exact bf16 products (error <= gamma_128 sum_e |q_e k_e|),
    scaled by the fp32 constant log2(e)/sqrt(128) into the log2 domain (a relative error u),
    one fused multiply-add and one v_exp_f32 (<= 4u relative) per term, row sums of the
    softmax denominator over chains of at most `depth` fp32 additions and a log2f, then a
    column sum of R = G w probabilities over RT + 4 additions and one division.  With
    eps_rj = ln2 (|d arg_rj| + |d LSE_r|) + 4u the relative error of p_rj, the bound is
    (1/R) sum_r p_rj eps_rj + imp_j (gamma_{RT+4} + u).  Returns ({g: exact imp}, {g: bound})."""
    w = q_obs.shape[0]
    n = K.shape[0]
    G = Hq // Hkv
    R = G * w
    nblk = -(-n // 512)                       # 512-key blocks
    P = min(256 // Hkv, nblk)                 # pass blocks per KV head
    # rounding steps in a row's softmax denominator (each ~u, an exp2 rescale ~4u): per lane 16
    # key terms and one rescale per key block it walks, two lane merges, eight wave merges, then
    # the merge of the P pass blocks (4 quarters of P/4, then the quarters)
    depth = 22 * -(-nblk // P) + 20 + 80 + 10 * (P // 4 + 4)
    qf = (np.ascontiguousarray(q_obs, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    imps, bounds = {}, {}
    for g in groups:
        kf = (np.ascontiguousarray(K[:, g, :], np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rows = qf[:, g * G:(g + 1) * G, :].transpose(1, 0, 2).reshape(R, D)
        arows = np.abs(rows)
        # pass 1: row maxima and sums (exact), and the worst relative error of a row's terms
        m = np.full(R, -np.inf)
        for j0 in range(0, n, chunk):
            m = np.maximum(m, (rows @ kf[j0:j0 + chunk].T).max(axis=1) / np.sqrt(D))
        l = np.zeros(R)
        term = np.zeros(R)
        for j0 in range(0, n, chunk):
            s = rows @ kf[j0:j0 + chunk].T / np.sqrt(D)
            a = arows @ np.abs(kf[j0:j0 + chunk]).T
            x = s * LOG2E
            dx = (LOG2E / np.sqrt(D)) * 128 * U * a + 2 * U * np.abs(x) + U * np.abs(x - m[:, None] * LOG2E)
            l += np.exp(s - m[:, None]).sum(axis=1)
            term = np.maximum(term, (np.log(2) * dx).max(axis=1))
        lse2 = (m + np.log(l)) * LOG2E
        dlse = (term + 4 * U + depth * U) / np.log(2) + 2 * U * np.abs(lse2)
        imp = np.zeros(n)
        eb = np.zeros(n)
        for j0 in range(0, n, chunk):
            s = rows @ kf[j0:j0 + chunk].T / np.sqrt(D)
            a = arows @ np.abs(kf[j0:j0 + chunk]).T
            arg = s * LOG2E - lse2[:, None]
            pr = np.exp2(arg)
            darg = (LOG2E / np.sqrt(D)) * 128 * U * a + U * np.abs(s * LOG2E) + U * np.abs(arg) + dlse[:, None]
            eps = np.log(2) * darg + 4 * U
            imp[j0:j0 + chunk] = pr.mean(axis=0)
            eb[j0:j0 + chunk] = (pr * eps).mean(axis=0)
        rt = R // 16
        imps[g] = imp
        bounds[g] = eb + imp * ((rt + 4) * U + U)
    return imps, bounds


def pooled_bound(imp, imp_bound):
    """Bound of |gpu pooled - exact pooled|: the three taps' importance bounds averaged, plus
    the rounding of two fp32 additions and one division (4u of the pooled value)."""
    out = {}
    for g, eb in imp_bound.items():
        pad = np.concatenate([[0.0], eb, [0.0]])
        pi = np.concatenate([[0.0], imp[g], [0.0]])
        pooled = (pi[:-2] + pi[1:-1] + pi[2:]) / 3.0
        out[g] = (pad[:-2] + pad[1:-1] + pad[2:]) / 3.0 + 4 * U * pooled
    return out


def check_snap_endtoend(x, r, groups=None):
    """SnapKV top-c end to end: the GPU lists against the oracle's top-c of the oracle's pooled
    importance.  Every token in which a KV head's lists differ must have an oracle pooled value
    within 1e-5 relative of the oracle boundary value, plus the derived error bound of the GPU
    pooled values at that token and at the boundary token as a floor."""
    Hq, Hkv = x.Hq, x.Hkv
    n = x.K.shape[0]
    groups = list(range(Hkv)) if groups is None else list(groups)
    if n <= 20000:
        full = O.snapkv_importance(x.q_obs, x.K, Hq, Hkv)
        imp = {g: full[g] for g in groups}
    else:
        imp = O.snapkv_importance_matmul(x.q_obs, x.K, Hq, Hkv, groups=groups)
    _, eb = snap_importance_bound(x.q_obs, x.K, Hq, Hkv, groups)
    pb = pooled_bound(imp, eb)
    idx = r["idx"].cpu().numpy()
    ndiff, worst, within_rel = 0, 0.0, True
    for g in groups:
        pooled = O.avg_pool1d(imp[g][None], 3)[0]
        sel_o = O.topc(pooled[None], x.c)[0]
        kap_t = min(sel_o, key=lambda t: (pooled[t], -t))
        kap = pooled[kap_t]
        tol = REL * np.maximum(pooled, kap) + pb[g] + pb[g][kap_t]
        d, w = _boundary_diff(idx[g], sel_o, pooled, lambda t: False, tol)
        ndiff += d
        worst = max(worst, w)
        within_rel &= w <= REL
    return {"diff_tokens": ndiff, "worst_rel_from_boundary": worst, "swaps_within_1e-5": bool(within_rel)}
