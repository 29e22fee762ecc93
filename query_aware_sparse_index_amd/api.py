"""Python binding of the qasi C ABI (argument marshalling only).

Every function takes torch tensors that live on the HIP device, passes their raw pointers
and the current stream to libqasi.so, and returns the tensors the library wrote.  Torch is
used for device memory and streams; every step of the computation runs in the library's
gfx950 kernels.  bf16 tensors may be torch.bfloat16 or int16/uint16 bit patterns.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

MODE_VOTE = 0
MODE_PER_HEAD = 1
MODE_UNION = 2          # decode_workspace_bytes only: the workspace of union_decode
MODE_DENSE = 3          # tiered_decode only: every position of each sequence


class QasiError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"qasi error {code}: {msg}")
        self.code = code


def _check(rc: int):
    if rc != 0:
        raise QasiError(rc, _lib.load().ts_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _p(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _host_i64(arr):
    a = (ctypes.c_int64 * len(arr))(*[int(x) for x in arr])
    return a


def _bf16_check(*ts):
    for t in ts:
        if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError(f"expected bf16 bits, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def params(mode=MODE_VOTE, budget=(1, 5), sink=4, local=256, v_min=1, theta=(9, 10)) -> _lib.SelectParams:
    return _lib.SelectParams(mode, 0, int(budget[0]), int(budget[1]), int(sink), int(local), int(v_min),
                             int(theta[0]), int(theta[1]))


def budget_tokens(n: int, p: _lib.SelectParams) -> int:
    return int(_lib.load().ts_budget_tokens(int(n), ctypes.byref(p)))


class Offsets:
    """Sequence offsets held twice, on the device (for kernels) and on the host (for sizing)."""

    def __init__(self, offsets, device="cuda"):
        self.host_list = [int(x) for x in offsets]
        self.host = _host_i64(self.host_list)
        self.dev = torch.tensor(self.host_list, dtype=torch.int64, device=device)
        self.B = len(self.host_list) - 1
        self.ntot = self.host_list[-1]


def index_append(k_new, P, k_index, pos: int):
    _bf16_check(k_new, k_index)
    T, Hkv, _ = k_new.shape
    _check(_lib.load().ts_index_append(_p(k_new), _p(P), _p(k_index), int(pos), int(T), int(Hkv), _stream()))
    return k_index


def score_stride(offs: Offsets) -> int:
    return int(_lib.load().ts_score_stride(offs.host, offs.B))


def score_workspace_bytes(B: int, Hq: int) -> int:
    return int(_lib.load().ts_score_workspace_bytes(int(B), int(Hq)))


def score(q, P, k_index, offs: Offsets, Hkv: int, out=None, ws=None):
    """Returns the [Hq][S] score array (row stride S = score_stride(offs) >= Ntot)."""
    _bf16_check(q, k_index)
    Hq = q.shape[1]
    if out is None:
        out = torch.empty((Hq, score_stride(offs)), dtype=torch.float32, device=q.device)
    need = score_workspace_bytes(offs.B, Hq)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(_lib.load().ts_score(_p(q), _p(P), _p(k_index), _p(offs.dev), offs.host, offs.B, Hq, int(Hkv),
                                _p(out), _p(ws), ws.numel(), _stream()))
    return out


def select_workspace_bytes(offs: Offsets, Hq: int, p) -> int:
    return int(_lib.load().ts_select_workspace_bytes(offs.host, offs.B, int(Hq), ctypes.byref(p)))


def select(scores, offs: Offsets, Hkv: int, p, want_theta=False, want_votes=False, ws=None, idx=None, count=None):
    Hq = scores.shape[0]
    ks = [budget_tokens(offs.host_list[b + 1] - offs.host_list[b], p) for b in range(offs.B)]
    total = sum(ks) * (Hq if p.mode == MODE_PER_HEAD else 1)
    dev = scores.device
    if idx is None:
        idx = torch.empty(max(total, 4), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty(offs.B, dtype=torch.int64, device=dev)
    theta = torch.empty((offs.B, Hq), dtype=torch.float32, device=dev) if want_theta else None
    votes = torch.empty(max(offs.ntot, 16), dtype=torch.uint8, device=dev) if want_votes else None
    need = select_workspace_bytes(offs, Hq, p)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(_lib.load().ts_select(_p(scores), _p(offs.dev), offs.host, offs.B, Hq, int(Hkv), ctypes.byref(p),
                                 _p(idx), _p(count), _p(theta), _p(votes), _p(ws), ws.numel(), _stream()))
    res = {"idx": idx[:total], "count": count, "counts_host": ks}
    if want_theta:
        res["theta"] = theta
    if want_votes:
        res["votes"] = votes[:offs.ntot]
    return res


def score_select_workspace_bytes(offs: Offsets, Hq: int, p) -> int:
    return int(_lib.load().ts_score_select_workspace_bytes(offs.host, offs.B, int(Hq), ctypes.byref(p)))


def score_select(q, P, k_index, offs: Offsets, Hkv: int, p, K_last=None, want_theta=False, want_votes=False,
                 ws=None, scores=None, idx=None, count=None):
    """ts_score followed by ts_select in one call (same outputs); with K_last, the index row of
    every sequence's last token is appended from the K cache first.  Returns the select() dict
    plus "scores"."""
    _bf16_check(q, k_index)
    if K_last is not None:
        _bf16_check(K_last)
    Hq = q.shape[1]
    dev = q.device
    ks = [budget_tokens(offs.host_list[b + 1] - offs.host_list[b], p) for b in range(offs.B)]
    total = sum(ks) * (Hq if p.mode == MODE_PER_HEAD else 1)
    if scores is None:
        scores = torch.empty((Hq, score_stride(offs)), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(max(total, 4), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty(offs.B, dtype=torch.int64, device=dev)
    theta = torch.empty((offs.B, Hq), dtype=torch.float32, device=dev) if want_theta else None
    votes = torch.empty(max(offs.ntot, 16), dtype=torch.uint8, device=dev) if want_votes else None
    need = score_select_workspace_bytes(offs, Hq, p)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(_lib.load().ts_score_select(_p(q), _p(P), _p(k_index), _p(K_last), _p(offs.dev), offs.host, offs.B, Hq,
                                       int(Hkv), ctypes.byref(p), _p(scores), _p(idx), _p(count), _p(theta),
                                       _p(votes), _p(ws), ws.numel(), _stream()))
    res = {"idx": idx[:total], "count": count, "counts_host": ks, "scores": scores}
    if want_theta:
        res["theta"] = theta
    if want_votes:
        res["votes"] = votes[:offs.ntot]
    return res


def score_select_state(ws, offs: Offsets, Hq: int, p):
    """ts_score_select_state_offset: the per-(sequence, head) records that a completed
    score_select call left in its workspace `ws`, as an int64 view [B, Hq, 8] (flag, answer key,
    keys above, need, bracket lo, bracket hi, range begin, range end)."""
    off = int(_lib.load().ts_score_select_state_offset(offs.host, offs.B, int(Hq), ctypes.byref(p)))
    if off < 0:
        raise ValueError(_lib.load().ts_last_error().decode())
    n = offs.B * int(Hq) * 8 * 8
    return ws[off:off + n].view(torch.int64).view(offs.B, int(Hq), 8)


def expand_capacity(k_prev: int, n: int, sink=4, local=256, radius=1) -> int:
    return int(_lib.load().ts_expand_capacity(int(k_prev), int(n), int(sink), int(local), int(radius)))


def expand_selection(idx_prev, counts_prev_dev, counts_prev_host, offs: Offsets, lists: int = 1, sink=4, local=256,
                     radius=1, out=None, caps=None, valid=None, ws=None):
    """ts_expand_selection: the previous lists widened by +-radius plus the current forced tokens,
    padded with -1 to their capacities.  Returns a dict with "idx", "caps" (device), "caps_host",
    "valid" (device [B][lists])."""
    dev = idx_prev.device
    caps_host = [expand_capacity(counts_prev_host[b], offs.host_list[b + 1] - offs.host_list[b], sink, local, radius)
                 for b in range(offs.B)]
    if out is None:
        out = torch.empty(max(lists * sum(caps_host), 4), dtype=torch.int32, device=dev)
    if caps is None:
        caps = torch.empty(offs.B, dtype=torch.int64, device=dev)
    if valid is None:
        valid = torch.empty((offs.B, lists), dtype=torch.int64, device=dev)
    ch = _host_i64(counts_prev_host)
    need = int(_lib.load().ts_expand_workspace_bytes(ch, offs.B, int(lists)))
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(_lib.load().ts_expand_selection(_p(idx_prev), _p(counts_prev_dev), ch, _p(offs.dev), offs.host, offs.B,
                                           int(lists), int(sink), int(local), int(radius), _p(out), _p(caps),
                                           _p(valid), _p(ws), ws.numel(), _stream()))
    return {"idx": out[:lists * sum(caps_host)], "caps": caps, "caps_host": caps_host, "valid": valid}


def decode_workspace_bytes(offs: Offsets, counts_host, Hq: int, Hkv: int, mode: int) -> int:
    ch = _host_i64(counts_host) if counts_host is not None else None
    return int(_lib.load().ts_decode_workspace_bytes(offs.host, ch, offs.B, int(Hq), int(Hkv), int(mode)))


def sparse_decode(q, K, V, offs: Offsets, idx, counts_dev, counts_host, mode: int, ws=None, out=None):
    _bf16_check(q, K, V)
    B, Hq, _ = q.shape
    Hkv = K.shape[1]
    if out is None:
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(offs, counts_host, Hq, Hkv, mode)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(_lib.load().ts_sparse_decode(_p(q), _p(K), _p(V), _p(offs.dev), offs.host, _p(idx), _p(counts_dev),
                                        _host_i64(counts_host), int(mode), B, Hq, Hkv, _p(out), _p(ws), ws.numel(),
                                        _stream()))
    return out


def sparse_decode_timed(q, K, V, offs: Offsets, idx, counts_dev, counts_host, mode: int, ws=None, out=None):
    """ts_sparse_decode_timed: sparse_decode, waiting for it; returns (out, the gather kernel's
    duration in microseconds from its dispatch timestamps)."""
    _bf16_check(q, K, V)
    B, Hq, _ = q.shape
    Hkv = K.shape[1]
    if out is None:
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(offs, counts_host, Hq, Hkv, mode)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    us = ctypes.c_float()
    _check(_lib.load().ts_sparse_decode_timed(_p(q), _p(K), _p(V), _p(offs.dev), offs.host, _p(idx), _p(counts_dev),
                                              _host_i64(counts_host), int(mode), B, Hq, Hkv, _p(out), _p(ws),
                                              ws.numel(), _stream(), ctypes.byref(us)))
    return out, float(us.value)


def sparse_decode_noalloc(q, K, V, offs: Offsets, idx, counts_dev, counts_host, mode: int, out=None):
    """ts_sparse_decode_noalloc: sparse_decode with the partials in the library's static device
    scratch (no workspace argument).  Calls on one device must not overlap."""
    _bf16_check(q, K, V)
    B, Hq, _ = q.shape
    Hkv = K.shape[1]
    if out is None:
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device=q.device)
    _check(_lib.load().ts_sparse_decode_noalloc(_p(q), _p(K), _p(V), _p(offs.dev), offs.host, _p(idx),
                                                _p(counts_dev), _host_i64(counts_host), int(mode), B, Hq, Hkv,
                                                _p(out), _stream()))
    return out


def union_lists(idx, counts_dev, counts_host, offs: Offsets, Hq: int, Hkv: int, uidx=None, umask=None, ucount=None,
                ws=None):
    """ts_union_lists: per (sequence, KV head) the ascending union of the G per-head lists, the
    per-entry head masks and the union sizes.  Returns (uidx, umask, ucount [B][Hkv])."""
    dev = idx.device
    total = int(Hq) * sum(int(c) for c in counts_host)
    if uidx is None:
        uidx = torch.empty(max(total, 4), dtype=torch.int32, device=dev)
    if umask is None:
        umask = torch.empty(max(total, 16), dtype=torch.uint8, device=dev)
    if ucount is None:
        ucount = torch.empty((offs.B, int(Hkv)), dtype=torch.int64, device=dev)
    need = int(_lib.load().ts_union_workspace_bytes(offs.host, offs.B, int(Hkv)))
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(_lib.load().ts_union_lists(_p(idx), _p(counts_dev), _host_i64(counts_host), _p(offs.dev), offs.host, offs.B,
                                      int(Hq), int(Hkv), _p(uidx), _p(umask), _p(ucount), _p(ws), ws.numel(),
                                      _stream()))
    return uidx[:total], umask[:total], ucount


def union_decode(q, K, V, offs: Offsets, uidx, umask, ucount, counts_dev, counts_host, ws=None, out=None):
    """ts_union_decode: the per-head decode of the lists a union was built from, each K/V row of
    a group's union gathered once for its G heads."""
    _bf16_check(q, K, V)
    B, Hq, _ = q.shape
    Hkv = K.shape[1]
    if out is None:
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(offs, counts_host, Hq, Hkv, MODE_UNION)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(_lib.load().ts_union_decode(_p(q), _p(K), _p(V), _p(offs.dev), offs.host, _p(uidx), _p(umask), _p(ucount),
                                       _p(counts_dev), _host_i64(counts_host), B, Hq, Hkv, _p(out), _p(ws),
                                       ws.numel(), _stream()))
    return out


def dense_decode(q, K, V, offs: Offsets, ws=None, out=None):
    _bf16_check(q, K, V)
    B, Hq, _ = q.shape
    Hkv = K.shape[1]
    if out is None:
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(offs, None, Hq, Hkv, MODE_VOTE)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(_lib.load().ts_dense_decode(_p(q), _p(K), _p(V), _p(offs.dev), offs.host, B, Hq, Hkv, _p(out), _p(ws),
                                       ws.numel(), _stream()))
    return out


def host_device_pointer(t) -> int:
    """ts_host_device_pointer: the address kernels use for a pinned host tensor."""
    if t.device.type != "cpu" or not t.is_pinned():
        raise ValueError("expected a pinned host tensor")
    d = ctypes.c_void_p()
    _check(_lib.load().ts_host_device_pointer(ctypes.c_void_p(t.data_ptr()), ctypes.byref(d)))
    return int(d.value)


def tiered_decode(q, K_main, V_main, K_ring, V_ring, offs: Offsets, mode: int, idx=None, counts_dev=None,
                  counts_host=None, ws=None, out=None):
    """ts_tiered_decode: K_main / V_main [Ntot][Hkv][128] on the device or pinned on the host (the
    offloaded tier), K_ring / V_ring device [B][N][Hkv][128] holding each sequence's newest N
    positions at slot t mod N.  mode: MODE_VOTE / MODE_PER_HEAD (with idx and counts) or
    MODE_DENSE."""
    _bf16_check(q, K_main, V_main, K_ring, V_ring)
    B, Hq, _ = q.shape
    N, Hkv = K_ring.shape[1], K_ring.shape[2]
    dense = mode == MODE_DENSE
    if out is None:
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(offs, None if dense else counts_host, Hq, Hkv, MODE_VOTE if dense else mode)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)

    def addr(t):
        return ctypes.c_void_p(host_device_pointer(t) if t.device.type == "cpu" else t.data_ptr())

    _check(_lib.load().ts_tiered_decode(_p(q), addr(K_main), addr(V_main), _p(K_ring), _p(V_ring), int(N), _p(offs.dev),
                                        offs.host, _p(idx), _p(counts_dev),
                                        None if dense else _host_i64(counts_host), int(mode), B, Hq, Hkv, _p(out),
                                        _p(ws), ws.numel(), _stream()))
    return out


def snapkv_workspace_bytes(n: int, w: int, Hq: int, Hkv: int, c: int) -> int:
    return int(_lib.load().snapkv_workspace_bytes(int(n), int(w), int(Hq), int(Hkv), int(c)))


def snapkv_compress(q_obs, K, V, c: int = 4096, pool_kernel: int = 3, want_importance=False, ws=None):
    _bf16_check(q_obs, K, V)
    w, Hq, _ = q_obs.shape
    n, Hkv, _ = K.shape
    ce = min(c, n)
    dev = K.device
    idx = torch.empty((Hkv, ce), dtype=torch.int32, device=dev)
    K_out = torch.empty((ce, Hkv, 128), dtype=K.dtype, device=dev)
    V_out = torch.empty((ce, Hkv, 128), dtype=V.dtype, device=dev)
    imp = torch.empty((Hkv, n), dtype=torch.float32, device=dev) if want_importance else None
    pooled = torch.empty((Hkv, n), dtype=torch.float32, device=dev) if want_importance else None
    need = snapkv_workspace_bytes(n, w, Hq, Hkv, c)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(_lib.load().snapkv_compress(_p(q_obs), _p(K), _p(V), int(n), int(w), int(Hq), int(Hkv), int(c),
                                       int(pool_kernel), _p(idx), _p(K_out), _p(V_out), _p(imp), _p(pooled), _p(ws),
                                       ws.numel(), _stream()))
    res = {"idx": idx, "K": K_out, "V": V_out}
    if want_importance:
        res["importance"] = imp
        res["pooled"] = pooled
    return res


def snapkv_retain_clusters(idx, K, V, k_cluster: int = 1):
    """Cluster-based retention of snapkv_compress's lists idx [Hkv][ce]: widened by +-k_cluster,
    padded with -1, rows gathered (zero rows for the padding).  Returns idx, K, V, valid."""
    _bf16_check(K, V)
    n, Hkv, _ = K.shape
    ce = idx.shape[1]
    cap = expand_capacity(ce, n, 0, 0, k_cluster)
    dev = K.device
    io = torch.empty((Hkv, max(cap, 1)), dtype=torch.int32, device=dev)
    Ko = torch.empty((max(cap, 1), Hkv, 128), dtype=K.dtype, device=dev)
    Vo = torch.empty((max(cap, 1), Hkv, 128), dtype=V.dtype, device=dev)
    valid = torch.empty(Hkv, dtype=torch.int64, device=dev)
    need = int(_lib.load().snapkv_clusters_workspace_bytes(int(ce), int(Hkv)))
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(_lib.load().snapkv_retain_clusters(_p(idx), int(n), int(Hkv), int(ce), int(k_cluster), _p(K), _p(V),
                                              _p(io), _p(Ko), _p(Vo), _p(valid), _p(ws), ws.numel(), _stream()))
    return {"idx": io[:, :cap], "K": Ko[:cap], "V": Vo[:cap], "valid": valid}
