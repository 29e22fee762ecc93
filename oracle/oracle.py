"""ctypes wrapper over the plain fp64 CPU oracle in ``qasi_oracle.c``.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the CPU
baseline leg of the benchmark, never by the GPU library or its Python binding.  It
shares no code with the GPU path.  Arrays are NumPy; bf16 tensors travel as uint16 bit
patterns.  Every function cites the passage of the pages that defines it in the C file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qasi_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int

D = 128
DP = 32


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, default rounding)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.qo_bf16_round.restype = ctypes.c_uint16
        L.qo_bf16_round.argtypes = [ctypes.c_double]
        L.qo_bf16_widen.restype = ctypes.c_double
        L.qo_bf16_widen.argtypes = [ctypes.c_uint16]
        L.qo_index_project.restype = None
        L.qo_index_project.argtypes = [_u16p, _f32p, _i64, _int, _u16p, _vp, _vp]
        L.qo_score.restype = None
        L.qo_score.argtypes = [_u16p, _f32p, _u16p, _i64p, _int, _int, _int, _f64p]
        L.qo_theta_rank.restype = _i64
        L.qo_theta_rank.argtypes = [_i64, _i64, _i64]
        L.qo_theta.restype = None
        L.qo_theta.argtypes = [_f64p, _i64p, _int, _int, _i64, _i64, _f64p]
        L.qo_votes.restype = None
        L.qo_votes.argtypes = [_f64p, _f64p, _i64p, _int, _int, _i32p]
        L.qo_budget_tokens.restype = _i64
        L.qo_budget_tokens.argtypes = [_i64, _i64, _i64, _i64, _i64]
        L.qo_select_vote.restype = None
        L.qo_select_vote.argtypes = [_i32p, _i64p, _int, _i64, _i64, _i64, _i64, _i64, _i32p, _i64p]
        L.qo_select_per_head.restype = None
        L.qo_select_per_head.argtypes = [_f64p, _i64p, _int, _int, _i64, _i64, _i64, _i64, _i32p, _i64p]
        L.qo_decode.restype = None
        L.qo_decode.argtypes = [_u16p, _u16p, _u16p, _i64p, _i32p, _i64p, _int, _int, _int, _int, _f64p]
        L.qo_dense_decode.restype = None
        L.qo_dense_decode.argtypes = [_u16p, _u16p, _u16p, _i64p, _int, _int, _int, _f64p]
        L.qo_snapkv_importance.restype = None
        L.qo_snapkv_importance.argtypes = [_u16p, _u16p, _i64, _int, _int, _int, _f64p]
        L.qo_avg_pool1d.restype = None
        L.qo_avg_pool1d.argtypes = [_f64p, _i64, _i64, _int, _f64p]
        L.qo_topc.restype = _i64
        L.qo_topc.argtypes = [_f64p, _i64, _i64, _i64, _i32p]
        L.qo_expand_capacity.restype = _i64
        L.qo_expand_capacity.argtypes = [_i64, _i64, _i64, _i64, _i64]
        L.qo_expand_selection.restype = None
        L.qo_expand_selection.argtypes = [_i32p, _i64p, _i64p, _int, _int, _i64, _i64, _i64, _i32p, _i64p]
        L.qo_snapkv_retain_clusters.restype = _i64
        L.qo_snapkv_retain_clusters.argtypes = [_u16p, _u16p, _i64, _int, _i32p, _i64, _i64, _i32p, _u16p, _u16p,
                                                _i64p]
        L.qo_gather_rows.restype = None
        L.qo_gather_rows.argtypes = [_u16p, _u16p, _i64, _int, _i32p, _i64, _u16p, _u16p]
        L.qo_union_lists.restype = None
        L.qo_union_lists.argtypes = [_i32p, _i64p, _i64p, _int, _int, _int, _i32p, _u8p, _i64p]
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ scalars

def bf16_round(x: float) -> int:
    return int(lib().qo_bf16_round(float(x)))


def bf16_widen(bits: int) -> float:
    return float(lib().qo_bf16_widen(int(bits)))


def theta_rank(n: int, num: int, den: int) -> int:
    return int(lib().qo_theta_rank(n, num, den))


def budget_tokens(n: int, bnum: int, bden: int, sink: int, local: int) -> int:
    return int(lib().qo_budget_tokens(n, bnum, bden, sink, local))


# ------------------------------------------------------------------- stages

def index_project(k: np.ndarray, P: np.ndarray, with_exact: bool = False):
    """k: uint16 [T][Hkv][128]; P: float32 [128][32] -> uint16 [T][Hkv][32]."""
    k = _c(k, np.uint16)
    T, Hkv, d = k.shape
    assert d == D
    out = np.empty((T, Hkv, DP), np.uint16)
    ex = np.empty((T, Hkv, DP), np.float64) if with_exact else None
    mg = np.empty((T, Hkv, DP), np.float64) if with_exact else None
    lib().qo_index_project(k, _c(P, np.float32), T, Hkv, out,
                           ex.ctypes.data if with_exact else None,
                           mg.ctypes.data if with_exact else None)
    return (out, ex, mg) if with_exact else out


def score(q, P, k_index, offsets, Hq, Hkv):
    """q: uint16 [B][Hq][128]; k_index: uint16 [Ntot][Hkv][32] -> float64 [Hq][Ntot]."""
    offsets = _c(offsets, np.int64)
    B = len(offsets) - 1
    out = np.empty((Hq, int(offsets[-1])), np.float64)
    lib().qo_score(_c(q, np.uint16).reshape(-1), _c(P, np.float32), _c(k_index, np.uint16).reshape(-1),
                   offsets, B, Hq, Hkv, out)
    return out


def theta(scores, offsets, num=9, den=10):
    """scores: float64 [Hq][Ntot] -> float64 [B][Hq]."""
    offsets = _c(offsets, np.int64)
    B = len(offsets) - 1
    Hq = scores.shape[0]
    out = np.empty((B, Hq), np.float64)
    lib().qo_theta(_c(scores, np.float64), offsets, B, Hq, num, den, out)
    return out


def votes(scores, theta_, offsets):
    offsets = _c(offsets, np.int64)
    B = len(offsets) - 1
    Hq = scores.shape[0]
    out = np.empty(int(offsets[-1]), np.int32)
    lib().qo_votes(_c(scores, np.float64), _c(theta_, np.float64), offsets, B, Hq, out)
    return out


def select_vote(votes_, offsets, bnum, bden, sink=4, local=256, vmin=1):
    """-> (idx int32 [sum_b K_b], count int64 [B])."""
    offsets = _c(offsets, np.int64)
    B = len(offsets) - 1
    ks = [budget_tokens(int(offsets[b + 1] - offsets[b]), bnum, bden, sink, local) for b in range(B)]
    idx = np.empty(max(sum(ks), 1), np.int32)
    cnt = np.empty(B, np.int64)
    lib().qo_select_vote(_c(votes_, np.int32), offsets, B, bnum, bden, sink, local, vmin, idx, cnt)
    return idx[:sum(ks)], cnt


def select_per_head(scores, offsets, bnum, bden, sink=4, local=256):
    """-> (idx int32 [sum_b Hq*K_b], count int64 [B])."""
    offsets = _c(offsets, np.int64)
    B = len(offsets) - 1
    Hq = scores.shape[0]
    ks = [budget_tokens(int(offsets[b + 1] - offsets[b]), bnum, bden, sink, local) for b in range(B)]
    idx = np.empty(max(Hq * sum(ks), 1), np.int32)
    cnt = np.empty(B, np.int64)
    lib().qo_select_per_head(_c(scores, np.float64), offsets, B, Hq, bnum, bden, sink, local, idx, cnt)
    return idx[:Hq * sum(ks)], cnt


def decode(q, K, V, offsets, idx, count, mode, Hq, Hkv):
    """mode 0 (shared list per sequence) or 1 (list per query head) -> float64 [B][Hq][128]."""
    offsets = _c(offsets, np.int64)
    B = len(offsets) - 1
    out = np.empty((B, Hq, D), np.float64)
    idx = _c(idx, np.int32)
    if idx.size == 0:
        idx = np.zeros(1, np.int32)
    lib().qo_decode(_c(q, np.uint16).reshape(-1), _c(K, np.uint16).reshape(-1), _c(V, np.uint16).reshape(-1),
                    offsets, idx, _c(count, np.int64), mode, B, Hq, Hkv, out)
    return out


def dense_decode(q, K, V, offsets, Hq, Hkv):
    offsets = _c(offsets, np.int64)
    B = len(offsets) - 1
    out = np.empty((B, Hq, D), np.float64)
    lib().qo_dense_decode(_c(q, np.uint16).reshape(-1), _c(K, np.uint16).reshape(-1), _c(V, np.uint16).reshape(-1),
                          offsets, B, Hq, Hkv, out)
    return out


def snapkv_importance(q_obs, K, Hq, Hkv):
    """q_obs: uint16 [w][Hq][128]; K: uint16 [n][Hkv][128] -> float64 [Hkv][n]."""
    w = q_obs.shape[0]
    n = K.shape[0]
    out = np.empty((Hkv, n), np.float64)
    lib().qo_snapkv_importance(_c(q_obs, np.uint16).reshape(-1), _c(K, np.uint16).reshape(-1), n, w, Hq, Hkv, out)
    return out


def avg_pool1d(x, kernel=3):
    x = _c(x, np.float64)
    rows, n = x.shape
    out = np.empty_like(x)
    lib().qo_avg_pool1d(x, rows, n, kernel, out)
    return out


def topc(pooled, c):
    pooled = _c(pooled, np.float64)
    rows, n = pooled.shape
    ce = min(c, n)
    idx = np.empty((rows, max(ce, 1)), np.int32)
    lib().qo_topc(pooled, rows, n, c, idx)
    return idx[:, :ce]


def gather_rows(K, V, idx):
    n, Hkv, d = K.shape
    idx = _c(idx, np.int32)
    ce = idx.shape[1]
    Ko = np.empty((ce, Hkv, d), np.uint16)
    Vo = np.empty((ce, Hkv, d), np.uint16)
    lib().qo_gather_rows(_c(K, np.uint16), _c(V, np.uint16), n, Hkv, idx, ce, Ko, Vo)
    return Ko, Vo


def snapkv(q_obs, K, V, Hq, Hkv, c=4096, kernel=3):
    """Whole prefill-end compression: importance, pooled, indices, compacted K and V."""
    imp = snapkv_importance(q_obs, K, Hq, Hkv)
    pooled = avg_pool1d(imp, kernel)
    idx = topc(pooled, c)
    Ko, Vo = gather_rows(K, V, idx)
    return imp, pooled, idx, Ko, Vo


def snapkv_importance_matmul(q_obs, K, Hq, Hkv, groups=None):
    """The same importance as qo_snapkv_importance, with NumPy fp64 matmul as the QK^T step
    (for full-size checks where the plain loops are too slow).  Returns {g: imp[n]}."""
    w = q_obs.shape[0]
    G = Hq // Hkv
    qf = (np.ascontiguousarray(q_obs, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = {}
    for g in (range(Hkv) if groups is None else groups):
        kf = (np.ascontiguousarray(K[:, g, :], np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rows = qf[:, g * G:(g + 1) * G, :].transpose(1, 0, 2).reshape(G * w, D)
        s = rows @ kf.T / np.sqrt(D)
        s -= s.max(axis=1, keepdims=True)
        np.exp(s, out=s)
        s /= s.sum(axis=1, keepdims=True)
        out[g] = s.mean(axis=0)
    return out


def expand_capacity(k_prev, n, sink=4, local=256, radius=1):
    return int(lib().qo_expand_capacity(int(k_prev), int(n), int(sink), int(local), int(radius)))


def expand_selection(prev, counts_prev, offsets, lists=1, sink=4, local=256, radius=1):
    """Selection reuse with neighbour fetch: every list of `prev` (ts_select layout, `lists` lists
    per sequence with lengths counts_prev) widened by +-radius, joined with the current forced
    tokens, ascending, padded with -1 to the capacity.  Returns (idx, counts [B][lists], caps)."""
    offsets = _c(offsets, np.int64)
    counts_prev = _c(counts_prev, np.int64)
    B = len(offsets) - 1
    caps = [expand_capacity(counts_prev[b], offsets[b + 1] - offsets[b], sink, local, radius) for b in range(B)]
    out = np.empty(max(lists * sum(caps), 1), np.int32)
    cnt = np.empty(B * lists, np.int64)
    prev = _c(prev, np.int32)
    if prev.size == 0:
        prev = np.zeros(1, np.int32)
    lib().qo_expand_selection(prev, counts_prev, offsets, B, lists, sink, local, radius, out, cnt)
    return out[:lists * sum(caps)], cnt.reshape(B, lists), caps


def snapkv_retain_clusters(K, V, idx, k_cluster):
    """Cluster-based retention: idx [Hkv][ce] widened by +-k_cluster, padded with -1, and the rows
    gathered (zero rows for the padding).  Returns (idx_out [Hkv][cap], K_out, V_out, valid [Hkv])."""
    K = _c(K, np.uint16)
    V = _c(V, np.uint16)
    n, Hkv, _ = K.shape
    idx = _c(idx, np.int32)
    ce = idx.shape[1]
    cap = expand_capacity(ce, n, 0, 0, k_cluster)
    io = np.empty((Hkv, max(cap, 1)), np.int32)
    Ko = np.empty((max(cap, 1), Hkv, D), np.uint16)
    Vo = np.empty((max(cap, 1), Hkv, D), np.uint16)
    valid = np.empty(Hkv, np.int64)
    lib().qo_snapkv_retain_clusters(K, V, n, Hkv, idx, ce, k_cluster, io, Ko, Vo, valid)
    return io[:, :cap], Ko[:cap], Vo[:cap], valid


def union_lists(idx, count, offsets, Hq, Hkv):
    """Per-KV-group union of per-head lists (select_per_head's layout).  Returns (uidx, umask,
    ucount [B][Hkv]): for sequence b and KV head g, the block of G*k_b entries at
    Hq*kpre_b + g*G*k_b holds the union's tokens in ascending order, then -1; umask bit hh marks
    the tokens head g*G+hh selected."""
    offsets = _c(offsets, np.int64)
    count = _c(count, np.int64)
    B = len(offsets) - 1
    total = Hq * int(count.sum())
    idx = _c(idx, np.int32)
    if idx.size == 0:
        idx = np.zeros(1, np.int32)
    uidx = np.empty(max(total, 1), np.int32)
    umask = np.empty(max(total, 1), np.uint8)
    ucount = np.empty(B * Hkv, np.int64)
    lib().qo_union_lists(idx, count, offsets, B, Hq, Hkv, uidx, umask, ucount)
    return uidx[:total], umask[:total], ucount.reshape(B, Hkv)
