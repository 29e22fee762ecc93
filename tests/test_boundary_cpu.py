"""The C-ABI library loads, exports every function include/qasi.h declares, and rejects
invalid or unsupported calls synchronously, before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from query_aware_sparse_index_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(4096)          # aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p(4097)           # misaligned


def header_functions():
    txt = open(os.path.join(ROOT, "include", "qasi.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", txt, flags=re.M)))


def test_exports_match_header():
    lib = _lib.load()
    names = header_functions()
    assert len(names) == 28, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def _offs(vals):
    return (ctypes.c_int64 * len(vals))(*vals)


def _params(mode=0, bnum=1, bden=5, sink=4, local=256, vmin=1, tn=9, td=10):
    return _lib.SelectParams(mode, 0, bnum, bden, sink, local, vmin, tn, td)


def err():
    return _lib.load().ts_last_error().decode()


def test_score_stride():
    L = _lib.load()
    assert L.ts_score_stride(_offs([0, 131073]), 1) == 131136
    assert L.ts_score_stride(_offs([0, 64, 128]), 2) == 128
    assert L.ts_score_stride(None, 1) == -1


def test_budget_helper():
    L = _lib.load()
    p = _params()
    assert L.ts_budget_tokens(131072, ctypes.byref(p)) == 26214
    assert L.ts_budget_tokens(100, ctypes.byref(p)) == 100
    bad = _params(bden=0)
    assert L.ts_budget_tokens(100, ctypes.byref(bad)) == -1


def test_index_append_validation():
    L = _lib.load()
    assert L.ts_index_append(None, FAKE, FAKE, 0, 1, 8, None) == -1
    assert L.ts_index_append(MIS, FAKE, FAKE, 0, 1, 8, None) == -1
    assert L.ts_index_append(FAKE, FAKE, FAKE, -1, 1, 8, None) == -1
    assert L.ts_index_append(FAKE, FAKE, FAKE, 0, 1, 3, None) == -2
    assert L.ts_index_append(FAKE, FAKE, FAKE, 0, 0, 8, None) == 0   # nothing to do, no HIP call


@pytest.mark.parametrize("Hq,Hkv,code", [(32, 3, -2), (30, 8, -2), (24, 8, -2), (128, 8, -2), (0, 8, -1)])
def test_score_head_validation(Hq, Hkv, code):
    L = _lib.load()
    o = _offs([0, 100])
    assert L.ts_score(FAKE, FAKE, FAKE, FAKE, o, 1, Hq, Hkv, FAKE, FAKE, 1 << 20, None) == code
    assert err()


def test_offsets_validation():
    L = _lib.load()
    assert L.ts_score(FAKE, FAKE, FAKE, FAKE, _offs([1, 100]), 1, 32, 8, FAKE, FAKE, 1 << 20, None) == -1
    assert L.ts_score(FAKE, FAKE, FAKE, FAKE, _offs([0, 100, 50]), 2, 32, 8, FAKE, FAKE, 1 << 20, None) == -1
    assert L.ts_score(FAKE, FAKE, FAKE, FAKE, _offs([0, 100]), 0, 32, 8, FAKE, FAKE, 1 << 20, None) == -1
    p = _params()
    assert L.ts_select(FAKE, FAKE, _offs([0, 0]), 1, 32, 8, ctypes.byref(p), FAKE, FAKE, None, None, FAKE, 1 << 40,
                       None) == -1  # empty sequence


def test_score_workspace_validation():
    L = _lib.load()
    need = L.ts_score_workspace_bytes(1, 32)
    assert need >= 32 * 32 * 4
    assert L.ts_score_workspace_bytes(0, 32) == 0
    assert L.ts_score(FAKE, FAKE, FAKE, FAKE, _offs([0, 100]), 1, 32, 8, FAKE, FAKE, need - 1, None) == -3
    assert "workspace" in err()


def test_select_validation():
    L = _lib.load()
    o = _offs([0, 4096])
    for p, code in [(_params(mode=2), -1), (_params(bden=0), -1), (_params(tn=11, td=10), -1), (_params(sink=-1), -1),
                    (_params(vmin=-1), -1), (_params(tn=1, td=(1 << 31) + 1), -1), (_params(bnum=1, bden=(1 << 31) + 1), -1)]:
        assert L.ts_select(FAKE, FAKE, o, 1, 8, 2, ctypes.byref(p), FAKE, FAKE, None, None, FAKE, 1 << 40, None) == code
    p = _params()
    need = L.ts_select_workspace_bytes(o, 1, 8, ctypes.byref(p))
    assert need > 0
    assert L.ts_select(FAKE, FAKE, o, 1, 8, 2, ctypes.byref(p), FAKE, FAKE, None, None, FAKE, need - 1, None) == -3
    assert "workspace" in err()
    assert L.ts_select(FAKE, FAKE, o, 1, 8, 2, None, FAKE, FAKE, None, None, FAKE, need, None) == -1


def test_score_select_validation():
    L = _lib.load()
    o = _offs([0, 4096])
    args = lambda p, kl, ws: (FAKE, FAKE, FAKE, kl, FAKE, o, 1, 8, 2, ctypes.byref(p) if p else None, FAKE, FAKE, FAKE,
                              None, None, FAKE, ws, None)
    for p, code in [(_params(mode=2), -1), (_params(bden=0), -1), (_params(tn=11, td=10), -1), (_params(vmin=-1), -1)]:
        assert L.ts_score_select(*args(p, None, 1 << 40)) == code
    p = _params()
    assert L.ts_score_select(*args(None, None, 1 << 40)) == -1
    assert L.ts_score_select(*args(p, MIS, 1 << 40)) == -1
    need = L.ts_score_select_workspace_bytes(o, 1, 8, ctypes.byref(p))
    assert need > 0
    assert L.ts_score_select(*args(p, FAKE, need - 1)) == -3
    assert "workspace" in err()
    a = list(args(p, None, need))
    a[7], a[8] = 12, 8           # G = 1.5
    assert L.ts_score_select(*a) == -2
    a = list(args(p, None, need))
    a[5] = _offs([0, 10, 5])
    a[6] = 2
    assert L.ts_score_select(*a) == -1


def test_decode_validation():
    L = _lib.load()
    o = _offs([0, 1000])
    c_ok, c_bad0, c_big = _offs([100]), _offs([0]), _offs([1001])
    ws = 1 << 40
    assert L.ts_sparse_decode(FAKE, FAKE, FAKE, FAKE, o, FAKE, FAKE, c_bad0, 0, 1, 32, 8, FAKE, FAKE, ws, None) == -1
    assert L.ts_sparse_decode(FAKE, FAKE, FAKE, FAKE, o, FAKE, FAKE, c_big, 0, 1, 32, 8, FAKE, FAKE, ws, None) == -1
    assert L.ts_sparse_decode(FAKE, FAKE, FAKE, FAKE, o, FAKE, FAKE, c_ok, 7, 1, 32, 8, FAKE, FAKE, ws, None) == -1
    assert L.ts_sparse_decode(FAKE, FAKE, FAKE, FAKE, o, None, FAKE, c_ok, 0, 1, 32, 8, FAKE, FAKE, ws, None) == -1
    need = L.ts_decode_workspace_bytes(o, c_ok, 1, 32, 8, 0)
    assert L.ts_sparse_decode(FAKE, FAKE, FAKE, FAKE, o, FAKE, FAKE, c_ok, 0, 1, 32, 8, FAKE, FAKE, need - 1, None) == -3
    assert L.ts_dense_decode(FAKE, MIS, FAKE, FAKE, o, 1, 32, 8, FAKE, FAKE, ws, None) == -1
    need = L.ts_decode_workspace_bytes(o, None, 1, 32, 8, 0)
    assert L.ts_dense_decode(FAKE, FAKE, FAKE, FAKE, o, 1, 32, 8, FAKE, FAKE, need - 1, None) == -3


def test_decode_noalloc_validation():
    """The no-workspace decode validates like ts_sparse_decode and rejects calls whose workspace
    need exceeds its 64 MiB static scratch, all before any HIP call."""
    L = _lib.load()
    o = _offs([0, 1000])
    c_ok, c_bad0 = _offs([100]), _offs([0])
    assert L.ts_sparse_decode_noalloc(FAKE, FAKE, FAKE, FAKE, o, FAKE, FAKE, c_bad0, 0, 1, 32, 8, FAKE, None) == -1
    assert L.ts_sparse_decode_noalloc(FAKE, FAKE, FAKE, FAKE, o, FAKE, FAKE, c_ok, 7, 1, 32, 8, FAKE, None) == -1
    assert L.ts_sparse_decode_noalloc(MIS, FAKE, FAKE, FAKE, o, FAKE, FAKE, c_ok, 0, 1, 32, 8, FAKE, None) == -1
    assert L.ts_sparse_decode_noalloc(FAKE, FAKE, FAKE, FAKE, o, FAKE, FAKE, c_ok, 0, 1, 24, 8, FAKE, None) == -2
    # 2^20 list entries at 64 query heads: the partials' bound is far above 64 MiB
    big_o, big_c = _offs([0, 1 << 20]), _offs([1 << 20])
    assert L.ts_decode_workspace_bytes(big_o, big_c, 1, 64, 8, 0) > (64 << 20)
    assert L.ts_sparse_decode_noalloc(FAKE, FAKE, FAKE, FAKE, big_o, FAKE, FAKE, big_c, 0, 1, 64, 8, FAKE, None) == -3
    assert "static scratch" in err()


def test_snapkv_validation():
    L = _lib.load()
    ws = 1 << 40
    args = lambda n, w, Hq, Hkv, c, k: (FAKE, FAKE, FAKE, n, w, Hq, Hkv, c, k, FAKE, FAKE, FAKE, None, None, FAKE, ws, None)
    assert L.snapkv_compress(*args(1000, 32, 64, 8, 4096, 5)) == -2
    assert L.snapkv_compress(*args(1000, 3, 64, 8, 4096, 3)) == -2      # G*w = 24
    assert L.snapkv_compress(*args(1000, 64, 64, 8, 4096, 3)) == -2     # G*w = 512
    assert L.snapkv_compress(*args(0, 32, 64, 8, 4096, 3)) == -1
    assert L.snapkv_compress(*args(1000, 32, 64, 8, 0, 3)) == -1
    # longer than the top-c selection supports: rejected before anything is enqueued
    assert L.snapkv_compress(*args((1 << 24) + 1, 32, 64, 8, 4096, 3)) == -2
    assert "2^24" in err()
    need = L.snapkv_workspace_bytes(1000, 32, 64, 8, 4096)
    assert need > 0
    a = list(args(1000, 32, 64, 8, 4096, 3))
    a[-2] = need - 1
    assert L.snapkv_compress(*a) == -3


def test_union_validation():
    """ts_union_lists / ts_union_decode reject bad pointers, head layouts, counts and short
    workspaces before any HIP call; the union decode's workspace query needs the counts."""
    L = _lib.load()
    o = _offs([0, 10000])
    c_ok, c_bad0, c_big = _offs([2000]), _offs([0]), _offs([10001])
    ws = 1 << 40
    u = lambda idx, ch, Hq, Hkv, uidx, um, uc, w, wsn: L.ts_union_lists(idx, FAKE, ch, FAKE, o, 1, Hq, Hkv, uidx, um,
                                                                       uc, w, wsn, None)
    assert u(None, c_ok, 32, 8, FAKE, FAKE, FAKE, FAKE, ws) == -1
    assert u(FAKE, c_ok, 32, 8, MIS, FAKE, FAKE, FAKE, ws) == -1
    assert u(FAKE, c_ok, 32, 8, FAKE, FAKE, MIS, FAKE, ws) == -1
    assert u(FAKE, c_bad0, 32, 8, FAKE, FAKE, FAKE, FAKE, ws) == -1
    assert u(FAKE, c_big, 32, 8, FAKE, FAKE, FAKE, FAKE, ws) == -1
    assert u(FAKE, c_ok, 48, 4, FAKE, FAKE, FAKE, FAKE, ws) == -2          # G = 12 > 8 mask bits
    need = L.ts_union_workspace_bytes(o, 1, 8)
    assert need > 0 and L.ts_union_workspace_bytes(o, 0, 8) == 0
    assert u(FAKE, c_ok, 32, 8, FAKE, FAKE, FAKE, FAKE, need - 1) == -3
    assert "workspace" in err()
    d = lambda ch, Hq, Hkv, uidx, wsn: L.ts_union_decode(FAKE, FAKE, FAKE, FAKE, o, uidx, FAKE, FAKE, FAKE, ch, 1, Hq,
                                                         Hkv, FAKE, FAKE, wsn, None)
    assert d(c_ok, 32, 8, None, ws) == -1
    assert d(c_bad0, 32, 8, FAKE, ws) == -1
    assert d(c_ok, 24, 8, FAKE, ws) == -2
    assert L.ts_decode_workspace_bytes(o, None, 1, 32, 8, 2) == 0           # union mode needs the counts
    assert L.ts_decode_workspace_bytes(o, c_ok, 1, 32, 8, 7) == 0
    need_u = L.ts_decode_workspace_bytes(o, c_ok, 1, 32, 8, 2)
    assert need_u > L.ts_decode_workspace_bytes(o, c_ok, 1, 32, 8, 1)      # G * count slots per group
    assert d(c_ok, 32, 8, FAKE, need_u - 1) == -3


def test_score_select_state_offset():
    """The bracket records sit inside the fused call's workspace, 256-byte aligned, with room for
    B * Hq records of 8 int64; invalid arguments give -1."""
    L = _lib.load()
    for offs, Hq in (([0, 131072], 32), ([0, 5000, 5001, 20000], 8), ([0, 1], 4)):
        o = _offs(offs)
        B = len(offs) - 1
        for mode in (0, 1):
            p = _params(mode)
            off = L.ts_score_select_state_offset(o, B, Hq, ctypes.byref(p))
            ws = L.ts_score_select_workspace_bytes(o, B, Hq, ctypes.byref(p))
            assert off >= 0 and off % 256 == 0 and off + B * Hq * 64 <= ws, (offs, Hq, mode, off, ws)
    o = _offs([0, 100])
    assert L.ts_score_select_state_offset(o, 0, 8, ctypes.byref(_params())) == -1
    assert L.ts_score_select_state_offset(o, 1, 8, ctypes.byref(_params(bden=0))) == -1
    assert L.ts_score_select_state_offset(None, 1, 8, ctypes.byref(_params())) == -1


def test_tiered_decode_validation():
    """ts_tiered_decode rejects a ring length that is not a power of two in [1, 2^20], the union
    mode, null or misaligned tier pointers and a short workspace before any HIP call;
    ts_host_device_pointer rejects null pointers."""
    L = _lib.load()
    o = _offs([0, 1000])
    c = (ctypes.c_int64 * 1)(200)

    def call(N=64, mode=0, Kr=FAKE, Vr=FAKE, Km=FAKE, ws_bytes=1 << 40, Hq=8, Hkv=2, idx=FAKE):
        return L.ts_tiered_decode(FAKE, Km, FAKE, Kr, Vr, N, FAKE, o, idx, FAKE, c, mode, 1, Hq, Hkv, FAKE, FAKE,
                                  ws_bytes, None)
    for N in (0, 3, 96, (1 << 20) * 2, -4):
        assert call(N=N) == -1, N
        assert "power of two" in err()
    assert call(mode=2) == -1                     # the union lists have their own decode
    assert call(mode=4) == -1
    assert call(Kr=None) == -1
    assert call(Vr=MIS) == -1
    assert call(Km=MIS) == -1
    assert call(Hq=24, Hkv=8) == -2
    assert call(idx=None) == -1                   # list modes need the lists
    assert call(ws_bytes=16) == -3
    assert call(mode=3, idx=None, ws_bytes=16) == -3   # dense: no lists, then the workspace check
    d = ctypes.c_void_p()
    assert L.ts_host_device_pointer(None, ctypes.byref(d)) == -1
    assert L.ts_host_device_pointer(FAKE, None) == -1


def test_sparse_decode_timed_validation():
    """ts_sparse_decode_timed validates like ts_sparse_decode, and needs somewhere to put the time."""
    L = _lib.load()
    o = _offs([0, 1000])
    c = (ctypes.c_int64 * 1)(200)
    t = ctypes.c_float()

    def call(gus=ctypes.byref(t), mode=0, ws_bytes=1 << 40, K=FAKE, cnt=c):
        return L.ts_sparse_decode_timed(FAKE, K, FAKE, FAKE, o, FAKE, FAKE, cnt, mode, 1, 8, 2, FAKE, FAKE, ws_bytes,
                                        None, gus)
    assert call(gus=None) == -1
    assert call(mode=2) == -1
    assert call(K=MIS) == -1
    assert call(cnt=(ctypes.c_int64 * 1)(1001)) == -1
    assert call(ws_bytes=16) == -3
