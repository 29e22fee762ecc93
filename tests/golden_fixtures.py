"""Readers for the hand-checked fixtures under tests/golden/ (see each file's header for the
passage it follows)."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line


def page_parameters():
    params, budgets = {}, []
    for line in _lines("page_parameters.txt"):
        if line.startswith("budget "):
            kv = dict(tok.split("=") for tok in line.split()[1:])
            budgets.append((int(kv["n"]), int(kv["K"])))
        else:
            k, v = (s.strip() for s in line.split("="))
            params[k] = int(v)
    return params, budgets


def _sel_args(tokens):
    kv = dict(t.split("=") for t in tokens)
    num, den = (int(x) for x in kv["budget"].split("/"))
    return int(kv["sink"]), int(kv["local"]), num, den, int(kv.get("vmin", 1))


def vote_example():
    """-> dict(scores [3][12] float64, theta [3], votes [12], selects [(sink, local, num, den,
    vmin, idx)], perhead {h: (sink, local, num, den, idx)}, union {"tokens"|"masks": (sink, local,
    num, den, values)})."""
    scores, out = [], {"selects": [], "perhead": {}, "union": {}}
    for line in _lines("vote_worked_example.txt"):
        lhs, rhs = line.split("->") if "->" in line else (line, None)
        if lhs.startswith("scores"):
            scores.append([float(x) for x in lhs.split("=")[1].split()])
        elif lhs.startswith("theta"):
            out["theta"] = np.array([float(x) for x in lhs.split("=")[1].split()])
        elif lhs.startswith("votes"):
            out["votes"] = np.array([int(x) for x in lhs.split("=")[1].split()], np.int32)
        elif lhs.startswith("select"):
            sink, local, num, den, vmin = _sel_args(lhs.split()[1:])
            out["selects"].append((sink, local, num, den, vmin, np.array([int(x) for x in rhs.split()], np.int32)))
        elif lhs.startswith("perhead"):
            toks = lhs.split()
            sink, local, num, den, _ = _sel_args(toks[1:-1])
            out["perhead"][int(toks[-1][1:])] = (sink, local, num, den, np.array([int(x) for x in rhs.split()], np.int32))
        elif lhs.startswith("union"):
            toks = lhs.split()
            sink, local, num, den, _ = _sel_args(toks[1:-1])
            out["union"][toks[-1]] = (sink, local, num, den, np.array([int(x) for x in rhs.split()], np.int64))
    out["scores"] = np.array(scores, np.float64)
    return out


def pool_example():
    imp, pooled, tops = None, None, []
    for line in _lines("pool_topc_example.txt"):
        if line.startswith("importance"):
            imp = np.array([float(x) for x in line.split("=")[1].split()])
        elif line.startswith("pooled"):
            pooled = np.array([float(a) / float(b) for a, b in (t.split("/") for t in line.split("=")[1].split())])
        elif line.startswith("topc"):
            lhs, rhs = line.split("->")
            tops.append((int(lhs.split("=")[1]), np.array([int(x) for x in rhs.split()], np.int32)))
    return imp, pooled, tops


def expand_example():
    """The worked neighbour-fetch example: n, sink, local, prev and per radius (valid, padding)."""
    vals, cases = {}, []
    for line in open(os.path.join(GOLDEN, "expand_example.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("radius"):
            head, rest = line.split("->")
            valid, pad = rest.split("|")
            cases.append((int(head.split()[1]), [int(x) for x in valid.split()], [int(x) for x in pad.split()]))
        else:
            k, v = line.split("=")
            vals[k.strip()] = [int(x) for x in v.split()]
    return vals["n"][0], vals["sink"][0], vals["local"][0], np.array(vals["prev"], np.int32), cases
