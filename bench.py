"""Decode-step benchmark: query-aware selection + sparse attention on one MI355X.

Workload: one LLaMA-3-8B-shaped attention layer (32 query / 8 KV heads, d = 128, index
d' = 32) with n = 131072 cached tokens, a 20 % selection budget and voting mode.  A step is
the whole hot path: the index row of the step's new key, the index scores, the selection
and the sparse decode, with the cache, the index and the step's query already resident in
HBM.  By default (--path fused) it is ts_score_select (which appends the index row itself)
+ ts_sparse_decode; --path calls runs ts_index_append + ts_score + ts_select +
ts_sparse_decode instead (the same outputs; reported beside the headline either way).  The last-level
cache is flushed (a 512 MiB read) before every timed step, outside the timed region, so
the figure is HBM-cold.  Time is measured with HIP events on the stream the kernels run on.

Prints one JSON line (see the fields below); --out also writes it to a file.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0       # MI355X HBM3E peak
METRIC = "µs/decode step + HBM GB/s (% peak), 128K ctx, 20% budget, 1 MI355X"


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
DECODE_SRC = os.path.join(ROOT, "query_aware_sparse_index_amd", "csrc", "decode.hip")


def measured_traffic(mode, n, budget):
    """HBM bytes per launch of the decode's gather kernel (decode_partial_kernel) from the
    committed counter measurement (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known
    size), or None when there is none for this workload or the decode source has changed since
    it was taken."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(DECODE_SRC, "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    for r in rec.get("records", []):
        if r.get("decode_hip_sha256") == digest and r.get("mode") == mode and r.get("budget") == budget:
            return r.get("gather_bytes_per_launch")
    return None


# ------------------------------------------------------------------ CPU oracle leg
# The oracle as it stands (plain fp64 C loops, one thread per step) on the host cores: whole
# decode steps of the benchmarked workload, first one after another in this process, then one
# step per worker process, all at once, on min(host cores, 16) processes.  It runs before the
# GPU is initialised, so the workers are plain forks sharing the inputs.
_CPU = {}


def _oracle_step(s):
    from oracle import oracle as O
    c = _CPU
    n = c["n0"] + s + 1
    kidx = np.concatenate([c["kidx"], O.index_project(c["K"][n - 1:n], c["P"])])
    o = np.array([0, n], np.int64)
    sc = O.score(c["Q"][s], c["P"], kidx, o, c["Hq"], c["Hkv"])
    if c["vote"]:
        th = O.theta(sc, o, 9, 10)
        il, cnt = O.select_vote(O.votes(sc, th, o), o, c["bnum"], c["bden"])
    else:
        il, cnt = O.select_per_head(sc, o, c["bnum"], c["bden"])
    O.decode(c["Q"][s], c["K"][:n], c["V"][:n], o, il, cnt, 0 if c["vote"] else 1, c["Hq"], c["Hkv"])
    return s


def cpu_baseline(x, Kh, Vh, Qh, n0, vote, bnum, bden, nseq):
    import multiprocessing as mp
    from oracle import oracle as O
    O.build()
    _CPU.update(n0=n0, K=Kh, V=Vh, Q=Qh, P=x.P, Hq=x.Hq, Hkv=x.Hkv, vote=vote, bnum=bnum, bden=bden)
    _CPU["kidx"] = O.index_project(Kh[:n0], x.P)
    t0 = time.perf_counter()
    for s in range(nseq):
        _oracle_step(s)
    one = (time.perf_counter() - t0) / nseq
    procs = max(1, min(os.cpu_count() or 1, 16))
    ctx = mp.get_context("fork")
    with ctx.Pool(procs) as pool:
        t0 = time.perf_counter()
        pool.map(_oracle_step, [i % len(Qh) for i in range(procs)], chunksize=1)
        wall = time.perf_counter() - t0
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(wall / procs * 1e6, 1), "unit": "us/step", "cores": procs, "kind": "oracle",
            "single_thread_us_per_step": round(one * 1e6, 1), "cpu_model": model,
            "sample": f"{procs} whole decode steps of the benchmarked workload (n={n0}+s, fp64 C oracle, one step per "
                      f"process on {procs} processes at once; value = wall time / steps) after {nseq} steps one "
                      f"after another in one process (single_thread_us_per_step); {os.cpu_count()} host cores visible"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--n", type=int, default=131072)
    ap.add_argument("--budget", type=int, default=20, help="percent (5, 10, 15, 20, 30)")
    ap.add_argument("--mode", choices=["vote", "per-head"], default="vote")
    ap.add_argument("--workload", choices=["long", "ragged", "snapkv", "offload"], default="long",
                    help="long: one sequence of --n tokens (the headline); ragged: a batch of 16 sequences of "
                         "16K-64K tokens at a 15%% budget; snapkv: SnapKV prefill-end compression alone "
                         "(LLaMA-3-70B layer shapes, n = --n, w = 32, c = 4096); offload: the --n-token layer with "
                         "its KV cache in pinned host memory and the newest --ring tokens in a device ring "
                         "(selection on the GPU, sparse against dense decode across the host link)")
    ap.add_argument("--ring", type=int, default=256, help="ring length of the offload workload (a power of two)")
    ap.add_argument("--path", choices=["fused", "calls"], default="fused",
                    help="fused: ts_score_select (with the index append) + ts_sparse_decode; calls: ts_index_append + "
                         "ts_score + ts_select + ts_sparse_decode")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip dense / warm / graph side measurements")
    ap.add_argument("--cpu-steps", type=int, default=3, help="oracle steps run one after another")
    ap.add_argument("--reuse-radius", type=int, nargs="+", default=[0, 1],
                    help="neighbour-fetch radii of the selection-reuse side measurement")
    ap.add_argument("--isolate", action="store_true", help="also time each call alone after a flush")
    ap.add_argument("--copy-probe", action="store_true",
                    help="end with three plain 256 MiB elementwise copies (torch.neg on fp32), a reference "
                         "for the HBM byte counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="no GPU: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, then "
                         "WRITE_SIZE, of a --copy-probe run) into the per-launch HBM traffic record")
    ap.add_argument("--out", default=None)
    return ap.parse_args()


PROBE_BYTES = 256 << 20


def traffic_record(fetch_csv, write_csv, out_path, mode=0, budget=20):
    """Per-launch HBM bytes of ts_sparse_decode from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by the factor that maps the probe copy's counter onto its known
    256 MiB.  Also returns a per-kernel table (mean KiB per dispatch, scaled bytes)."""
    import csv
    import hashlib

    def load(path, counter):
        rows = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return rows

    fetch = load(fetch_csv, "FETCH_SIZE")
    write = load(write_csv, "WRITE_SIZE")
    probe = lambda d: [v for k, vs in d.items() if "neg_kernel" in k for v in vs]
    pf, pw = probe(fetch), probe(write)
    if not pf or not pw:
        raise SystemExit("no probe copy (neg_kernel) in the counter files: run the profiled bench with --copy-probe")
    f_scale = (PROBE_BYTES / 1024.0) / float(np.median(pf))
    w_scale = (PROBE_BYTES / 1024.0) / float(np.median(pw))
    table = {}
    for k in sorted(set(fetch) | set(write)):
        fk = float(np.mean(fetch.get(k, [0.0])))
        wk = float(np.mean(write.get(k, [0.0])))
        table[k] = {"fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                    "bytes": int(1024 * (fk * f_scale + wk * w_scale))}
    dec = [k for k in table if "decode_partial_kernel" in k or "decode_merge_kernel" in k]
    gather = [k for k in dec if "decode_partial_kernel" in k]
    with open(DECODE_SRC, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    rec = {"bytes_per_launch": int(sum(table[k]["bytes"] for k in dec)),
           "gather_bytes_per_launch": int(sum(table[k]["bytes"] for k in gather)),
           "kernels": {k: table[k] for k in dec},
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "mode": mode, "budget": budget, "decode_hip_sha256": digest}
    # one record per (mode, budget): a new measurement replaces the old one of its workload
    try:
        with open(out_path) as f:
            old = json.load(f).get("records", [])
    except (OSError, ValueError):
        old = []
    recs = [r for r in old if (r.get("mode"), r.get("budget")) != (mode, budget)] + [rec]
    with open(out_path, "w") as f:
        json.dump({"records": recs}, f, indent=1)
        f.write("\n")
    return rec, table


def bench_ragged(args, torch, api, synth, dev):
    """Ragged batch (Mistral-7B layer shapes, 16 sequences of 16K-64K tokens, 15 % budget): a
    step appends the index row of each sequence's newest token (one ts_index_append per
    sequence), then ts_score + ts_select + ts_sparse_decode over the packed batch.  Inputs
    resident in HBM, LLC flushed before each step, events on the launch stream."""
    import ctypes
    from query_aware_sparse_index_amd import _lib
    L = _lib.load()
    mode = api.MODE_VOTE if args.mode == "vote" else api.MODE_PER_HEAD
    print("bench: building the ragged batch", file=sys.stderr, flush=True)
    x = synth.config4()
    Hq, Hkv = x.Hq, x.Hkv
    offs = api.Offsets(x.offsets, dev)
    lens = [int(v) for v in np.diff(x.offsets)]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    q, K, V = t(x.q), t(x.K), t(x.V)
    P = torch.from_numpy(x.P).to(dev)
    kidx = torch.empty((offs.ntot, Hkv, 32), dtype=torch.int16, device=dev)
    api.index_append(K, P, kidx, 0)
    p = api.params(mode, x.budget)
    ks = [api.budget_tokens(n, p) for n in lens]
    scores = torch.empty((Hq, api.score_stride(offs)), dtype=torch.float32, device=dev)
    idx = torch.empty(sum(ks) * (Hq if mode == api.MODE_PER_HEAD else 1) + 16, dtype=torch.int32, device=dev)
    count = torch.empty(offs.B, dtype=torch.int64, device=dev)
    ws_sc = torch.empty(max(api.score_workspace_bytes(offs.B, Hq), 256), dtype=torch.uint8, device=dev)
    ws_sel = torch.empty(max(api.select_workspace_bytes(offs, Hq, p), 256), dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(max(api.decode_workspace_bytes(offs, ks, Hq, Hkv, mode), 256), dtype=torch.uint8,
                         device=dev)
    out = torch.empty((offs.B, Hq, 128), dtype=torch.float32, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    vp = lambda a: ctypes.c_void_p(a.data_ptr())
    ch = (ctypes.c_int64 * offs.B)(*ks)
    Kp, Vp, Pp, kip, qp, scp = vp(K), vp(V), vp(P), vp(kidx), vp(q), vp(scores)
    row_bytes = Hkv * 128 * 2
    pref = ctypes.byref(p)

    def chk(rc):
        if rc != 0:
            raise RuntimeError(L.ts_last_error().decode())

    ws_ss = torch.empty(max(api.score_select_workspace_bytes(offs, Hq, p), 256), dtype=torch.uint8, device=dev)

    def step():
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if args.path == "fused":
            chk(L.ts_score_select(qp, Pp, kip, Kp, vp(offs.dev), offs.host, offs.B, Hq, Hkv, pref, scp, vp(idx),
                                  vp(count), None, None, vp(ws_ss), ws_ss.numel(), st))
        else:
            for b in range(offs.B):
                last = offs.host_list[b + 1] - 1
                chk(L.ts_index_append(ctypes.c_void_p(Kp.value + last * row_bytes), Pp, kip, last, 1, Hkv, st))
            chk(L.ts_score(qp, Pp, kip, vp(offs.dev), offs.host, offs.B, Hq, Hkv, scp, vp(ws_sc), ws_sc.numel(), st))
            chk(L.ts_select(scp, vp(offs.dev), offs.host, offs.B, Hq, Hkv, pref, vp(idx), vp(count), None, None,
                            vp(ws_sel), ws_sel.numel(), st))
        chk(L.ts_sparse_decode(qp, Kp, Vp, vp(offs.dev), offs.host, vp(idx), vp(count), ch, mode, offs.B, Hq, Hkv,
                               vp(out), vp(ws_dec), ws_dec.numel(), st))

    for _ in range(args.warmup):
        torch.sum(flush.view(torch.float32), dim=0, out=sink)
        step()
    torch.cuda.synchronize()
    evs = []
    for _ in range(args.steps):
        torch.sum(flush.view(torch.float32), dim=0, out=sink)
        a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b2.record()
        evs.append((a, b2))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b2) * 1e3 for a, b2 in evs])
    ntot = offs.ntot
    kv_rows = sum(ks) if mode == api.MODE_VOTE else None
    if kv_rows is None:       # per-head: union of each KV group's lists
        G = Hq // Hkv
        lst = idx[:sum(ks) * Hq].cpu().numpy()
        kv_rows, base = 0, 0
        for k in ks:
            blk = lst[base:base + Hq * k].reshape(Hq, k)
            kv_rows += sum(len(np.unique(blk[g * G:(g + 1) * G])) for g in range(Hkv))
            base += Hq * k
        step_bytes = ntot * Hkv * 64 + kv_rows * 128 * 2 * 2
    else:
        step_bytes = ntot * Hkv * 64 + kv_rows * Hkv * 128 * 2 * 2
    mean = float(us.mean())
    res = {"metric": METRIC, "value": round(mean, 2), "unit": "us/step", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(mean / 1e3, 5), "higher_is_better": False,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"ragged batch of {offs.B} sequences ({min(lens)}-{max(lens)} tokens, "
                                  f"{ntot} in total), 32 query / 8 KV heads, d=128, d'=32, budget "
                                  f"{x.budget[0]}/{x.budget[1]}, {args.mode} mode", "B": offs.B, "Ntot": ntot,
                      "path": args.path,
                      "llc": "flushed before each step"},
           "median_us": round(float(np.median(us)), 2),
           "hbm_gbps": round(step_bytes / (mean * 1e-6) / 1e9, 1),
           "pct_peak": round(100 * step_bytes / (mean * 1e-6) / 1e9 / PEAK_GBPS, 1),
           "algorithmic_bytes_per_step": int(step_bytes)}
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


def bench_snapkv(args, torch, api, synth, dev):
    """SnapKV prefill-end compression at LLaMA-3-70B layer shapes (64 query / 8 KV heads, d = 128,
    w = 32, c = 4096, pool 3) over n prompt tokens: --steps calls, the LLC flushed before each,
    events on the launch stream."""
    n = args.n
    print(f"bench: building SnapKV inputs n={n}", file=sys.stderr, flush=True)
    sx = synth.config5(n)
    qo, K, V = (torch.from_numpy(a.view(np.int16)).to(dev) for a in (sx.q_obs, sx.K, sx.V))
    ws = torch.empty(api.snapkv_workspace_bytes(n, 32, 64, 8, 4096), dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        torch.sum(flush.view(torch.float32), dim=0, out=sink)
        api.snapkv_compress(qo, K, V, 4096, ws=ws)
    torch.cuda.synchronize()
    evs = []
    for _ in range(args.steps):
        torch.sum(flush.view(torch.float32), dim=0, out=sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        api.snapkv_compress(qo, K, V, 4096, ws=ws)
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    mean = float(us.mean())
    flop_pass = 2.0 * 64 * 32 * n * 128
    byts = n * 8 * 128 * 2 + 2 * 4096 * 8 * 128 * 2 * 2
    res = {"metric": "µs per SnapKV compression (LLaMA-3-70B layer, w=32, c=4096), 1 MI355X", "value": round(mean, 2),
           "unit": "us/call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"SnapKV compress, Hq=64 Hkv=8 d=128 n={n} w=32 c=4096 pool 3", "n": n,
                      "llc": "flushed before each call"},
           "median_us": round(float(np.median(us)), 2),
           "mfma_tflops_executed": round(2 * flop_pass / (mean * 1e-6) / 1e12, 1),
           "mfma_frac_bf16_peak": round(2 * flop_pass / (mean * 1e-6) / 2.5e15, 4),
           "algorithmic_tflops": round(flop_pass / (mean * 1e-6) / 1e12, 1),
           "algorithmic_gbps": round(byts / (mean * 1e-6) / 1e9, 1)}
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


def bench_offload(args, torch, api, synth, dev):
    """The 128K-token layer (32 query / 8 KV heads) with the KV cache in pinned host memory, the
    newest --ring tokens in a device ring, the index on the device: per call, the GPU selection
    (ts_score_select), the sparse tiered decode of its list and the dense tiered decode, each timed
    alone (--steps calls, LLC flushed before each), plus the whole step (selection + sparse decode)
    and a plain host-to-device copy of 256 MiB as the host link's reference rate."""
    n, N = args.n, args.ring
    bnum, bden = synth.BUDGETS[args.budget]
    print(f"bench: building offload inputs n={n} ring={N} budget={bnum}/{bden}", file=sys.stderr, flush=True)
    x = synth.config3(args.budget, n)
    Hq, Hkv = x.Hq, x.Hkv
    mode = api.MODE_VOTE if args.mode == "vote" else api.MODE_PER_HEAD
    offs = api.Offsets(x.offsets, dev)
    Kh = torch.from_numpy(x.K.view(np.int16)).pin_memory()
    Vh = torch.from_numpy(x.V.view(np.int16)).pin_memory()

    def ring(a):
        # slot t mod N of the device ring holds position t of the newest N
        slots = np.empty((N,) + a.shape[1:], np.uint16)
        slots[np.arange(n - N, n) % N] = a[n - N:]
        return torch.from_numpy(slots.reshape(1, N, Hkv, 128).view(np.int16)).to(dev)

    Kr, Vr = ring(x.K), ring(x.V)
    P = torch.from_numpy(x.P).to(dev)
    kidx = torch.empty((n, Hkv, 32), dtype=torch.int16, device=dev)
    api.index_append(torch.from_numpy(x.K.view(np.int16)).to(dev), P, kidx, 0)
    q = torch.from_numpy(x.q.view(np.int16)).to(dev)
    p = api.params(mode, (bnum, bden))
    vote = mode == api.MODE_VOTE
    sel = api.score_select(q, P, kidx, offs, Hkv, p)
    ws_sel = torch.empty(api.score_select_workspace_bytes(offs, Hq, p), dtype=torch.uint8, device=dev)
    ch = sel["counts_host"]
    ws_dec = torch.empty(max(api.decode_workspace_bytes(offs, ch, Hq, Hkv, mode),
                             api.decode_workspace_bytes(offs, None, Hq, Hkv, api.MODE_VOTE)), dtype=torch.uint8, device=dev)
    out = torch.empty((1, Hq, 128), dtype=torch.float32, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def sparse():
        api.tiered_decode(q, Kh, Vh, Kr, Vr, offs, mode, sel["idx"], sel["count"], ch, ws=ws_dec, out=out)

    def dense():
        api.tiered_decode(q, Kh, Vh, Kr, Vr, offs, api.MODE_DENSE, ws=ws_dec, out=out)

    def step():
        s2 = api.score_select(q, P, kidx, offs, Hkv, p, ws=ws_sel, scores=sel["scores"], idx=sel["idx"],
                              count=sel["count"])
        api.tiered_decode(q, Kh, Vh, Kr, Vr, offs, mode, s2["idx"], s2["count"], ch, ws=ws_dec, out=out)

    def timed(fn, steps, warm):
        for _ in range(warm):
            torch.sum(flush.view(torch.float32), dim=0, out=sink)
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(steps):
            torch.sum(flush.view(torch.float32), dim=0, out=sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) * 1e3 for a, b in evs]))

    steps, warm = max(3, args.steps // 10), max(1, args.warmup // 5)
    us_sparse = timed(sparse, steps, warm)
    print(f"bench: sparse tiered decode {us_sparse:.1f} us", file=sys.stderr, flush=True)
    us_dense = timed(dense, max(2, steps // 2), 1)
    print(f"bench: dense tiered decode {us_dense:.1f} us", file=sys.stderr, flush=True)
    us_step = timed(step, steps, warm)
    # the host link's plain copy rate: 256 MiB of pinned host memory to the device
    hsrc = torch.empty(256 << 20, dtype=torch.uint8).pin_memory()
    ddst = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    us_copy = timed(lambda: ddst.copy_(hsrc, non_blocking=True), 3, 1)
    # vote mode: the list's rows older than the ring cross the host link (K and V of every KV head)
    idx_np = sel["idx"].cpu().numpy()
    rows_host = int((idx_np < n - N).sum()) if vote else None
    row_bytes = Hkv * 128 * 2 * 2
    res = {"metric": "µs per decode-step attention with the KV cache in host memory (128K ctx, 20% budget), 1 MI355X",
           "value": round(us_step, 2), "unit": "us/step", "n_gpus": 1, "steps": steps, "warmup": warm,
           "higher_is_better": False, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"LLaMA-3-8B-shaped decode layer, n={n}, 32 query / 8 KV heads, KV cache in pinned "
                                  f"host memory, newest {N} tokens in a device ring, {args.mode} mode, budget "
                                  f"{bnum}/{bden}", "n": n, "ring": N, "mode": args.mode, "llc": "flushed before each call"},
           "sparse_decode_us": round(us_sparse, 1), "dense_decode_us": round(us_dense, 1),
           "dense_over_sparse": round(us_dense / us_sparse, 2),
           "sparse_host_gbps": round(rows_host * row_bytes / (us_sparse * 1e-6) / 1e9, 1) if vote else None,
           "dense_host_gbps": round((n - N) * row_bytes / (us_dense * 1e-6) / 1e9, 1),
           "host_copy_gbps": round((256 << 20) / (us_copy * 1e-6) / 1e9, 1)}
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


def bench_union(torch, api, L, calls, warm, steps, Hq, Hkv, kmax, offs_max, Kp, Vp, Pp, kip, pref, scp, idp, cnp,
                wss, ws_ss_n, outp, out, ws_dec, dec_bytes, do_flush, stream_of, chk, dev):
    """Per-head lists decoded through their per-KV-group union: ts_score_select, ts_union_lists,
    ts_union_decode per step (LLC flushed before each step), the per-call split in separate steps,
    each union call alone, and the largest difference from ts_sparse_decode on the same lists."""
    import ctypes
    ev = lambda: torch.cuda.Event(enable_timing=True)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    un_idx = torch.empty(kmax * Hq + 16, dtype=torch.int32, device=dev)
    un_msk = torch.empty(kmax * Hq + 16, dtype=torch.uint8, device=dev)
    un_cnt = torch.empty((1, Hkv), dtype=torch.int64, device=dev)
    ws_un = torch.empty(max(int(L.ts_union_workspace_bytes(offs_max.host, 1, Hkv)), 256), dtype=torch.uint8,
                        device=dev)
    ws_ud = torch.empty(max(api.decode_workspace_bytes(offs_max, [kmax], Hq, Hkv, api.MODE_UNION), 256),
                        dtype=torch.uint8, device=dev)
    out_u = torch.empty_like(out)
    uip, ump, ucp, wup, wudp, oup = vp(un_idx), vp(un_msk), vp(un_cnt), vp(ws_un), vp(ws_ud), vp(out_u)

    def sel(s, st):
        (_, _), (qp, od, oh), ch, kb = calls[s]
        chk(L.ts_score_select(qp, Pp, kip, Kp, od, oh, 1, Hq, Hkv, pref, scp, idp, cnp, None, None, wss, ws_ss_n, st))

    def union(s, st):
        (_, _), (qp, od, oh), ch, kb = calls[s]
        chk(L.ts_union_lists(idp, cnp, ch, od, oh, 1, Hq, Hkv, uip, ump, ucp, wup, ws_un.numel(), st))

    def udec(s, st):
        (_, _), (qp, od, oh), ch, kb = calls[s]
        chk(L.ts_union_decode(qp, Kp, Vp, od, oh, uip, ump, ucp, cnp, ch, 1, Hq, Hkv, oup, wudp, ws_ud.numel(), st))

    nb = min(steps, 30)
    whole, parts = [], []
    for i in range(nb):
        do_flush()
        st = stream_of()
        a, b = ev(), ev()
        a.record()
        sel(warm + i, st)
        union(warm + i, st)
        udec(warm + i, st)
        b.record()
        whole.append((a, b))
    for i in range(nb):
        do_flush()
        st = stream_of()
        m = [ev() for _ in range(4)]
        m[0].record()
        sel(warm + i, st)
        m[1].record()
        union(warm + i, st)
        m[2].record()
        udec(warm + i, st)
        m[3].record()
        parts.append(m)
    torch.cuda.synchronize()
    alone = {}
    s_last = warm + steps - 1
    st = stream_of()
    sel(s_last, st)
    for name, fn in (("union_lists", union), ("union_decode", udec)):
        evs = []
        for r in range(12):
            do_flush()
            a, b = ev(), ev()
            a.record()
            fn(s_last, st)
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        alone[name] = round(float(np.mean([a.elapsed_time(b) * 1e3 for a, b in evs[2:]])), 2)
    (_, _), (qp, od, oh), ch, kb = calls[s_last]
    chk(L.ts_sparse_decode(qp, Kp, Vp, od, oh, idp, cnp, ch, api.MODE_PER_HEAD, 1, Hq, Hkv, outp, vp(ws_dec),
                           ws_dec.numel(), st))
    torch.cuda.synchronize()
    uc = un_cnt.cpu().numpy()
    return {"us_per_step": round(float(np.mean([a.elapsed_time(b) * 1e3 for a, b in whole])), 2),
            "breakdown_us": {nm: round(float(np.mean([m[k].elapsed_time(m[k + 1]) * 1e3 for m in parts])), 2)
                             for k, nm in enumerate(["score_select", "union_lists", "union_decode"])},
            "alone_us": alone,
            "union_rows_per_kv_head": round(float(uc.mean()), 1), "selected_per_head": int(kb),
            "union_decode_gbps": round(dec_bytes / (alone["union_decode"] * 1e-6) / 1e9, 1),
            "max_abs_diff_vs_sparse_decode": float((out_u - out).abs().max().item())}


def main():
    args = parse()
    if args.traffic_from:
        mode = 0 if args.mode == "vote" else 1
        rec, table = traffic_record(args.traffic_from[0], args.traffic_from[1], TRAFFIC_FILE, mode, args.budget)
        for k, v in table.items():
            print(f"{v['fetch_kib']:14.1f} {v['write_kib']:14.1f} {v['bytes'] / 1e6:10.2f} MB  {k[:90]}")
        print(json.dumps({k: v for k, v in rec.items() if k != "kernels"}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode-step path of one attention layer runs on a single "
              "MI355X (sharding across GPUs is not built); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from query_aware_sparse_index_amd import api, synth

    dev = torch.device("cuda:0")
    if args.workload == "ragged":
        return bench_ragged(args, torch, api, synth, dev)
    if args.workload == "snapkv":
        return bench_snapkv(args, torch, api, synth, dev)
    if args.workload == "offload":
        return bench_offload(args, torch, api, synth, dev)
    n0, steps, warm = args.n, args.steps, args.warmup
    total_steps = steps + warm
    mode = api.MODE_VOTE if args.mode == "vote" else api.MODE_PER_HEAD
    bnum, bden = synth.BUDGETS[args.budget]
    print(f"bench: building inputs n={n0} budget={bnum}/{bden} mode={args.mode} steps={steps} warmup={warm}",
          file=sys.stderr, flush=True)

    x = synth.config3(args.budget, n0)
    Hq, Hkv = x.Hq, x.Hkv
    cap = n0 + total_steps
    # host copies of the cache with room for the decode steps (the new rows are drawn per step)
    Kh = np.empty((cap, Hkv, 128), np.uint16)
    Vh = np.empty((cap, Hkv, 128), np.uint16)
    Kh[:n0], Vh[:n0] = x.K, x.V
    qs = []
    for s in range(total_steps):
        q_s, k_new, v_new = synth.config3_step(s + 1, x.q, Hkv)
        Kh[n0 + s], Vh[n0 + s] = k_new[0], v_new[0]
        qs.append(q_s)
    Qh = np.stack(qs)                                                   # [steps][1][Hq][128]
    cpu = None
    if not args.no_cpu:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(x, Kh, Vh, Qh, n0, mode == api.MODE_VOTE, bnum, bden, args.cpu_steps)
        print(f"bench: CPU oracle {cpu['single_thread_us_per_step']} us/step on one thread, {cpu['value']} us/step on "
              f"{cpu['cores']} processes", file=sys.stderr, flush=True)
    K = torch.from_numpy(Kh.view(np.int16)).to(dev)
    V = torch.from_numpy(Vh.view(np.int16)).to(dev)
    Q = torch.from_numpy(Qh.view(np.int16)).to(dev)
    P = torch.from_numpy(x.P).to(dev)
    kidx = torch.empty((cap, Hkv, 32), dtype=torch.int16, device=dev)
    api.index_append(K[:n0], P, kidx, 0)
    p = api.params(mode, (bnum, bden))
    offs = [api.Offsets([0, n0 + s + 1], dev) for s in range(total_steps)]
    nmax = cap
    scores = torch.empty((Hq, api.score_stride(offs[-1])), dtype=torch.float32, device=dev)
    kmax = api.budget_tokens(nmax, p)
    idx = torch.empty(kmax * (Hq if mode == api.MODE_PER_HEAD else 1) + 16, dtype=torch.int32, device=dev)
    count = torch.empty(1, dtype=torch.int64, device=dev)
    ws_sel = torch.empty(max(api.select_workspace_bytes(offs[-1], Hq, p), 256), dtype=torch.uint8, device=dev)
    ws_ss = torch.empty(max(api.score_select_workspace_bytes(offs[-1], Hq, p), 256), dtype=torch.uint8, device=dev)
    ws_sc = torch.empty(max(api.score_workspace_bytes(1, Hq), 256), dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(max(api.decode_workspace_bytes(offs[-1], [kmax], Hq, Hkv, mode), 256), dtype=torch.uint8,
                         device=dev)
    out = torch.empty((1, Hq, 128), dtype=torch.float32, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def do_flush():
        torch.sum(flush.view(torch.float32), dim=0, out=flush_sink)

    ev = lambda: torch.cuda.Event(enable_timing=True)

    # argument tuples for the four C-ABI calls of every step, built before timing so that
    # the host enqueues a step in a few microseconds
    import ctypes
    from query_aware_sparse_index_amd import _lib
    L = _lib.load()
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    pref = ctypes.byref(p)
    stream_of = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = []
    for s in range(total_steps):
        n = n0 + s + 1
        o = offs[s]
        kb = api.budget_tokens(n, p)
        ch = (ctypes.c_int64 * 1)(kb)
        qp = ctypes.c_void_p(Q[s].data_ptr())
        calls.append(((vp(K) .value + (n - 1) * Hkv * 128 * 2, n - 1),
                      (qp, vp(o.dev), o.host), ch, kb))
    Kp, Pp, kip, scp, idp, cnp = vp(K), vp(P), vp(kidx), vp(scores), vp(idx), vp(count)
    Vp, outp, wsp, wdp, wsc, wss = vp(V), vp(out), vp(ws_sel), vp(ws_dec), vp(ws_sc), vp(ws_ss)
    ws_sel_n, ws_dec_n, ws_sc_n, ws_ss_n = ws_sel.numel(), ws_dec.numel(), ws_sc.numel(), ws_ss.numel()

    def chk(rc):
        if rc != 0:
            raise RuntimeError(L.ts_last_error().decode())

    def step_calls(s, marks=None):
        """The four calls: ts_index_append, ts_score, ts_select, ts_sparse_decode."""
        (kaddr, pos), (qp, od, oh), ch, kb = calls[s]
        st = stream_of()
        chk(L.ts_index_append(ctypes.c_void_p(kaddr), Pp, kip, pos, 1, Hkv, st))
        if marks: marks[1].record()
        chk(L.ts_score(qp, Pp, kip, od, oh, 1, Hq, Hkv, scp, wsc, ws_sc_n, st))
        if marks: marks[2].record()
        chk(L.ts_select(scp, od, oh, 1, Hq, Hkv, pref, idp, cnp, None, None, wsp, ws_sel_n, st))
        if marks: marks[3].record()
        chk(L.ts_sparse_decode(qp, Kp, Vp, od, oh, idp, cnp, ch, mode, 1, Hq, Hkv, outp, wdp, ws_dec_n, st))
        return kb

    def step_fused(s, marks=None):
        """ts_score_select (appending the step's index row itself) + ts_sparse_decode."""
        (kaddr, pos), (qp, od, oh), ch, kb = calls[s]
        st = stream_of()
        chk(L.ts_score_select(qp, Pp, kip, Kp, od, oh, 1, Hq, Hkv, pref, scp, idp, cnp, None, None, wss, ws_ss_n, st))
        if marks: marks[1].record()
        chk(L.ts_sparse_decode(qp, Kp, Vp, od, oh, idp, cnp, ch, mode, 1, Hq, Hkv, outp, wdp, ws_dec_n, st))
        return kb

    step = step_fused if args.path == "fused" else step_calls

    # warm-up
    for s in range(warm):
        if not args.no_flush:
            do_flush()
        step(s)
    torch.cuda.synchronize()
    print("bench: warm-up done", file=sys.stderr, flush=True)

    # timed steps: one event pair per step; flushes between steps are not timed
    marks = [(ev(), ev()) for _ in range(steps)]
    ktot = []
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(steps):
        s = warm + i
        if not args.no_flush:
            do_flush()
        marks[i][0].record()
        ktot.append(step(s))
        marks[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    step_us = np.array([a.elapsed_time(b) * 1e3 for a, b in marks])
    print(f"bench: timed {steps} steps, mean {step_us.mean():.1f} us", file=sys.stderr, flush=True)

    # per-call breakdown in separate steps (the same inputs again): an event between two calls
    # idles the GPU for a few microseconds, so these steps are not the timed ones
    nb = min(steps, 30)
    names = ["score_select", "sparse_decode"] if args.path == "fused" else \
        ["index_append", "score", "select", "sparse_decode"]
    bmarks = [[ev() for _ in range(len(names) + 1)] for _ in range(nb)]
    for i in range(nb):
        if not args.no_flush:
            do_flush()
        m = bmarks[i]
        m[0].record()
        step(warm + steps - nb + i, m)
        m[-1].record()
    torch.cuda.synchronize()
    parts = {nm: np.array([m[k].elapsed_time(m[k + 1]) * 1e3 for m in bmarks]) for k, nm in enumerate(names)}
    breakdown_step = float(np.mean([m[0].elapsed_time(m[-1]) * 1e3 for m in bmarks]))

    # the other path (four separate calls, or the fused one) on the same steps, for reference
    other = step_calls if args.path == "fused" else step_fused
    omarks = [(ev(), ev()) for _ in range(nb)]
    for i in range(nb):
        if not args.no_flush:
            do_flush()
        omarks[i][0].record()
        other(warm + steps - nb + i)
        omarks[i][1].record()
    torch.cuda.synchronize()
    other_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in omarks]))

    # algorithmic bytes (what the method must move): index read + selected K/V rows
    n_mean = n0 + warm + (steps + 1) / 2.0
    k_mean = float(np.mean(ktot))
    if mode == api.MODE_VOTE:
        kv_bytes = k_mean * Hkv * 128 * 2 * 2          # one K and V row per KV head per selected token
    else:                                              # per KV head: the union of its heads' lists
        Gq = Hq // Hkv
        kl = int(ktot[-1])
        lst = idx[:kl * Hq].cpu().numpy().reshape(Hq, kl)
        kv_bytes = sum(len(np.unique(lst[g * Gq:(g + 1) * Gq])) for g in range(Hkv)) * 128 * 2 * 2
    idx_bytes = n_mean * Hkv * 32 * 2
    small = Hq * 128 * 2 + 128 * 32 * 4 + Hq * 128 * 4 + k_mean * 4
    step_bytes = idx_bytes + kv_bytes + small
    mean_us = float(step_us.mean())
    gbps = step_bytes / (mean_us * 1e-6) / 1e9

    # the dominant kernel alone: the decode's gather kernel (decode_partial_kernel), LLC flushed
    # before each launch, timed by its dispatch timestamps (ts_sparse_decode_timed: events
    # recorded by the kernel launch itself on the stream it runs on); the whole call (gather +
    # LSE merge + launch gap) by events around it, for reference; inputs of the last timed step
    s_last = warm + steps - 1
    (_, _), (qp_l, od_l, oh_l), ch_l, _ = calls[s_last]
    gather_us = []
    g_us = ctypes.c_float()
    for r in range(22):
        if not args.no_flush:
            do_flush()
        chk(L.ts_sparse_decode_timed(qp_l, Kp, Vp, od_l, oh_l, idp, cnp, ch_l, mode, 1, Hq, Hkv, outp, wdp, ws_dec_n,
                                     stream_of(), ctypes.byref(g_us)))
        gather_us.append(float(g_us.value))
    dec_us = float(np.mean(gather_us[2:]))
    dec_evs = []
    for r in range(22):
        if not args.no_flush:
            do_flush()
        st = stream_of()
        a, b2 = ev(), ev()
        a.record()
        chk(L.ts_sparse_decode(qp_l, Kp, Vp, od_l, oh_l, idp, cnp, ch_l, mode, 1, Hq, Hkv, outp, wdp, ws_dec_n, st))
        b2.record()
        dec_evs.append((a, b2))
    torch.cuda.synchronize()
    call_us = float(np.mean([a.elapsed_time(b2) * 1e3 for a, b2 in dec_evs[2:]]))
    k_last = float(ktot[-1])
    if mode == api.MODE_VOTE:
        dec_bytes = k_last * Hkv * 128 * 2 * 2 + Hq * 128 * 2 + k_last * 4
    else:
        # per-head lists: a KV head's rows are needed once for the union of its G heads' lists
        G = Hq // Hkv
        lists = idx[:int(k_last) * Hq].cpu().numpy().reshape(Hq, int(k_last))
        union_rows = sum(len(np.unique(lists[g * G:(g + 1) * G])) for g in range(Hkv))
        dec_bytes = union_rows * 128 * 2 * 2 + Hq * 128 * 2 + k_last * Hq * 4
    dec_gbps = dec_bytes / (dec_us * 1e-6) / 1e9
    traffic = measured_traffic(mode, n0 + warm + steps, args.budget)

    extra = {}
    if args.isolate:
        # each call alone: flush, event, call, event (inputs from the last timed step)
        s_iso = warm + steps - 1
        (kaddr, pos), (qp, od, oh), ch, kb = calls[s_iso]
        st = stream_of()
        iso_calls = {
            "index_append": lambda: chk(L.ts_index_append(ctypes.c_void_p(kaddr), Pp, kip, pos, 1, Hkv, st)),
            "score": lambda: chk(L.ts_score(qp, Pp, kip, od, oh, 1, Hq, Hkv, scp, wsc, ws_sc_n, st)),
            "select": lambda: chk(L.ts_select(scp, od, oh, 1, Hq, Hkv, pref, idp, cnp, None, None, wsp, ws_sel_n, st)),
            "sparse_decode": lambda: chk(L.ts_sparse_decode(qp, Kp, Vp, od, oh, idp, cnp, ch, mode, 1, Hq, Hkv, outp,
                                                            wdp, ws_dec_n, st)),
        }
        iso = {}
        for name, fn in iso_calls.items():
            for flushed in (True, False):
                evs = []
                for r in range(12):
                    if flushed:
                        do_flush()
                    a, b2 = ev(), ev()
                    a.record()
                    fn()
                    b2.record()
                    evs.append((a, b2))
                torch.cuda.synchronize()
                iso[f"{name}{'' if flushed else '_warm'}"] = round(float(np.mean([a.elapsed_time(b2) * 1e3 for a, b2 in evs[2:]])), 2)
        extra["isolated_us"] = iso
    if not args.no_extra:
        # measured device copy bandwidth: 1 GiB read + 1 GiB written per copy, events around 5 copies
        csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        cdst = torch.empty_like(csrc)
        cdst.copy_(csrc)
        cev = []
        for _ in range(5):
            a, b2 = ev(), ev()
            a.record()
            cdst.copy_(csrc)
            b2.record()
            cev.append((a, b2))
        torch.cuda.synchronize()
        copy_us = float(np.median([a.elapsed_time(b2) * 1e3 for a, b2 in cev]))
        extra["copy_gbps"] = round(2 * (1 << 30) / (copy_us * 1e-6) / 1e9, 1)
        del csrc, cdst
        # the two smaller decode configurations (tiny layer at 4K tokens, the 8B-shaped layer at 32K),
        # the same fused step (ts_score_select with the append, ts_sparse_decode), flushed, 20 steps
        cfgs = {}
        for name, xc in (("c1", synth.config1()), ("c2", synth.config2())):
            nc = int(xc.offsets[-1])
            oc = api.Offsets(xc.offsets, dev)
            qc, Kc, Vc = (torch.from_numpy(a.view(np.int16)).to(dev) for a in (xc.q, xc.K, xc.V))
            Pc = torch.from_numpy(xc.P).to(dev)
            kic = torch.empty((nc, xc.Hkv, 32), dtype=torch.int16, device=dev)
            api.index_append(Kc, Pc, kic, 0)
            pc = api.params(api.MODE_VOTE, xc.budget)
            kc = api.budget_tokens(nc, pc)
            wssc = torch.empty(api.score_select_workspace_bytes(oc, xc.Hq, pc), dtype=torch.uint8, device=dev)
            wsdc = torch.empty(api.decode_workspace_bytes(oc, [kc], xc.Hq, xc.Hkv, api.MODE_VOTE), dtype=torch.uint8,
                               device=dev)
            scc = torch.empty((xc.Hq, api.score_stride(oc)), dtype=torch.float32, device=dev)
            idc = torch.empty(kc + 16, dtype=torch.int32, device=dev)
            cnc = torch.empty(1, dtype=torch.int64, device=dev)
            outc = torch.empty((1, xc.Hq, 128), dtype=torch.float32, device=dev)
            pcr, chc = ctypes.byref(pc), (ctypes.c_int64 * 1)(kc)
            cevs = []
            for i in range(25):
                do_flush()
                st = stream_of()
                a, b2 = ev(), ev()
                a.record()
                chk(L.ts_score_select(vp(qc), vp(Pc), vp(kic), vp(Kc), vp(oc.dev), oc.host, 1, xc.Hq, xc.Hkv, pcr,
                                      vp(scc), vp(idc), vp(cnc), None, None, vp(wssc), wssc.numel(), st))
                chk(L.ts_sparse_decode(vp(qc), vp(Kc), vp(Vc), vp(oc.dev), oc.host, vp(idc), vp(cnc), chc,
                                       api.MODE_VOTE, 1, xc.Hq, xc.Hkv, vp(outc), vp(wsdc), wsdc.numel(), st))
                b2.record()
                cevs.append((a, b2))
            torch.cuda.synchronize()
            us = float(np.mean([a.elapsed_time(b2) * 1e3 for a, b2 in cevs[5:]]))
            byts = nc * xc.Hkv * 64 + kc * xc.Hkv * 512
            cfgs[name] = {"n": nc, "Hq": xc.Hq, "Hkv": xc.Hkv, "budget": f"{xc.budget[0]}/{xc.budget[1]}",
                          "us_per_step": round(us, 2), "algorithmic_bytes": int(byts),
                          "hbm_gbps": round(byts / (us * 1e-6) / 1e9, 1)}
        extra["configs"] = cfgs
        # dense flash-decode over all n under the same protocol
        n_d = n0
        od = api.Offsets([0, n_d], dev)
        ws_dd = torch.empty(max(api.decode_workspace_bytes(od, None, Hq, Hkv, api.MODE_VOTE), 256), dtype=torch.uint8,
                            device=dev)
        dts = []
        for i in range(20):
            do_flush()
            a, b = ev(), ev()
            a.record()
            api.dense_decode(Q[0], K, V, od, ws=ws_dd, out=out)
            b.record()
            dts.append((a, b))
        torch.cuda.synchronize()
        dense_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in dts[2:]]))
        extra["dense_decode_us"] = round(dense_us, 2)
        extra["dense_gbps"] = round(n_d * Hkv * 128 * 4 / (dense_us * 1e-6) / 1e9, 1)
        # warm last-level cache (no flush), same steps
        w_us = []
        for i in range(min(steps, 30)):
            a, b = ev(), ev()
            a.record()
            step(warm + i)
            b.record()
            w_us.append((a, b))
        torch.cuda.synchronize()
        extra["warm_llc_us"] = round(float(np.mean([a.elapsed_time(b) * 1e3 for a, b in w_us])), 2)
        # hipGraph capture of one step at a fixed n, replayed with flushes in between
        try:
            s_fix = warm
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                step(s_fix)
            torch.cuda.current_stream().wait_stream(cs)
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                step(s_fix)
            g_us = []
            for i in range(30):
                do_flush()
                a, b = ev(), ev()
                a.record()
                g.replay()
                b.record()
                g_us.append((a, b))
            torch.cuda.synchronize()
            extra["graph_step_us"] = round(float(np.mean([a.elapsed_time(b) * 1e3 for a, b in g_us[3:]])), 2)
        except Exception as e:  # capture is an optional side measurement
            extra["graph_step_us"] = f"unavailable: {type(e).__name__}"
        # selection reuse with neighbour fetch: the selector (ts_score_select) runs every N steps,
        # every step widens the last selection by +-radius and adds its forced tokens
        # (ts_expand_selection), then decodes the widened list; mean us per step over the same
        # flushed steps, for N = 1, 4, 8, 16
        lists = Hq if mode == api.MODE_PER_HEAD else 1
        cap_max = api.expand_capacity(kmax, nmax, 4, 256, max(args.reuse_radius))
        ex_idx = torch.empty(cap_max * lists + 16, dtype=torch.int32, device=dev)
        ex_caps = torch.empty(1, dtype=torch.int64, device=dev)
        ex_valid = torch.empty((1, lists), dtype=torch.int64, device=dev)
        ws_ex = torch.empty(max(api.decode_workspace_bytes(offs[-1], [cap_max], Hq, Hkv, mode), 256), dtype=torch.uint8,
                            device=dev)
        wsx = torch.empty(4096, dtype=torch.uint8, device=dev)      # chunk sums of the expansion
        exp_, capp, valp, wexp, wsxp = vp(ex_idx), vp(ex_caps), vp(ex_valid), vp(ws_ex), vp(wsx)
        extra["reuse"] = []
        for radius in args.reuse_radius:
            reuse = {"radius": radius, "us_per_step": {}}
            for N in (1, 4, 8, 16):
                r_evs, kprev = [], None
                for i in range(min(steps, 48)):
                    s_ = warm + i
                    (kaddr, pos), (qp, od, oh), ch, kb = calls[s_]
                    n_s = n0 + s_ + 1
                    do_flush()
                    st = stream_of()
                    a, b2 = ev(), ev()
                    a.record()
                    if i % N == 0:
                        chk(L.ts_score_select(qp, Pp, kip, Kp, od, oh, 1, Hq, Hkv, pref, scp, idp, cnp, None, None,
                                              wss, ws_ss_n, st))
                        kprev = (ctypes.c_int64 * 1)(kb)
                    chk(L.ts_expand_selection(idp, cnp, kprev, od, oh, 1, lists, 4, 256, radius, exp_, capp, valp,
                                              wsxp, wsx.numel(), st))
                    cap = api.expand_capacity(kprev[0], n_s, 4, 256, radius)
                    chk(L.ts_sparse_decode(qp, Kp, Vp, od, oh, exp_, capp, (ctypes.c_int64 * 1)(cap), mode, 1, Hq,
                                           Hkv, outp, wexp, ws_ex.numel(), st))
                    b2.record()
                    r_evs.append((a, b2))
                torch.cuda.synchronize()
                reuse["us_per_step"][str(N)] = round(float(np.mean([x.elapsed_time(y) * 1e3 for x, y in r_evs])), 2)
            reuse["mean_entries_per_list"] = round(float(ex_valid.float().mean().item()), 1)
            reuse["selected_per_list"] = int(kprev[0])
            extra["reuse"].append(reuse)
        if mode == api.MODE_PER_HEAD:
            extra["union"] = bench_union(torch, api, L, calls, warm, steps, Hq, Hkv, kmax, offs[-1], Kp, Vp, Pp, kip,
                                         pref, scp, idp, cnp, wss, ws_ss_n, outp, out, ws_dec, dec_bytes, do_flush,
                                         stream_of, chk, dev)
        # SnapKV prefill-end compression at LLaMA-3-70B layer shapes (64 / 8 heads, w = 32,
        # c = 4096, pool 3) over the same n, LLC flushed before each call
        sx = synth.config5(n0)
        qo_s, K_s, V_s = (torch.from_numpy(a.view(np.int16)).to(dev) for a in (sx.q_obs, sx.K, sx.V))
        ws_s = torch.empty(api.snapkv_workspace_bytes(n0, 32, 64, 8, 4096), dtype=torch.uint8, device=dev)
        api.snapkv_compress(qo_s, K_s, V_s, 4096, ws=ws_s)
        sts = []
        for i in range(12):
            do_flush()
            a, b = ev(), ev()
            a.record()
            api.snapkv_compress(qo_s, K_s, V_s, 4096, ws=ws_s)
            b.record()
            sts.append((a, b))
        torch.cuda.synchronize()
        snap_us = float(np.mean([a.elapsed_time(b) * 1e3 for a, b in sts[2:]]))
        flop_pass = 2.0 * 64 * 32 * n0 * 128                       # one Q_obs K^T over all keys
        snap_bytes = n0 * 8 * 128 * 2 + 2 * 4096 * 8 * 128 * 2 * 2   # K once + gather (read + write K, V)
        extra["snapkv"] = {"workload": f"Hq=64 Hkv=8 n={n0} w=32 c=4096 pool 3", "us": round(snap_us, 2),
                           "mfma_tflops_executed": round(2 * flop_pass / (snap_us * 1e-6) / 1e12, 1),
                           "mfma_frac_bf16_peak": round(2 * flop_pass / (snap_us * 1e-6) / 2.5e15, 4),
                           "algorithmic_tflops": round(flop_pass / (snap_us * 1e-6) / 1e12, 1),
                           "algorithmic_gbps": round(snap_bytes / (snap_us * 1e-6) / 1e9, 1)}
        del qo_s, K_s, V_s, ws_s

    res = {
        "metric": METRIC,
        "value": round(mean_us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(mean_us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"LLaMA-3-8B-shaped decode layer, n={n0} cached tokens, 32 query / 8 KV heads, "
                               f"d=128, d'=32, budget {args.budget}%, {args.mode} mode, sink 4 + local 256",
                   "n": n0, "Hq": Hq, "Hkv": Hkv, "budget": f"{bnum}/{bden}", "mode": args.mode,
                   "inputs": "bf16", "llc": "warm" if args.no_flush else "flushed before each step"},
        "median_us": round(float(np.median(step_us)), 2),
        "hbm_gbps": round(gbps, 1),
        "pct_peak": round(100 * gbps / PEAK_GBPS, 1),
        "algorithmic_bytes_per_step": int(step_bytes),
        "path": args.path,
        "breakdown_us": {k: round(float(v.mean()), 2) for k, v in parts.items()},
        "breakdown_step_us": round(breakdown_step, 2),
        ("four_call_step_us" if args.path == "fused" else "fused_step_us"): round(other_us, 2),
        "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps / PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "decode_partial_kernel (the gather of ts_sparse_decode), alone, LLC flushed, "
                               "timed by its dispatch timestamps",
                     "algorithmic_bytes": int(dec_bytes), "avg_us": round(dec_us, 2),
                     # the whole ts_sparse_decode call (gather + merge + launch gap), event-timed
                     "call_avg_us": round(call_us, 2),
                     "call_frac": round(dec_bytes / (call_us * 1e-6) / 1e9 / PEAK_GBPS, 4)},
        # the whole step (every call of the hot path) against the same peak: the metric's own figure
        "step_roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                          "frac": round(gbps / PEAK_GBPS, 4), "algorithmic_bytes": int(step_bytes),
                          "avg_us": round(mean_us, 2)},
        "cpu_baseline": cpu,
        "wall_s_timed_loop": round(wall, 4),
    }
    res.update(extra)
    if "copy_gbps" in extra:
        res["roofline"]["measured_copy_gbps"] = extra["copy_gbps"]
        res["roofline"]["frac_of_measured_copy"] = round(dec_gbps / extra["copy_gbps"], 4)
        res["step_roofline"]["frac_of_measured_copy"] = round(gbps / extra["copy_gbps"], 4)
    if args.copy_probe:
        src = torch.empty(PROBE_BYTES // 4, dtype=torch.float32, device=dev).fill_(3.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
    line = json.dumps(res)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
