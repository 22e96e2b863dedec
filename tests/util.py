"""Shared helpers of the test-suite (comparison metric, oracle adapters,
the pages' printed values under tests/golden/)."""
from pathlib import Path

import numpy as np

from oracle import model as om

# Parity bars: maximum relative error ||g - r||_inf / ||r||_inf against the
# float64 oracle run on the same (bf16-rounded where applicable) inputs.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(g, r):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if r.size == 0:
        return 0.0
    return float(np.max(np.abs(g - r)) / max(float(np.max(np.abs(r))), 1e-30))


def oracle_reqs(work, idx=None):
    idx = range(work.n_reqs) if idx is None else idx
    out, off = [], 0
    for i in idx:
        out.append(om.Req(off, work.q_len[i], work.kv_len[i]))
        off += work.q_len[i]
    return out


def f64_params(params):
    return [{k: np.asarray(v, dtype=np.float64) for k, v in p.items()} for p in params]


def f64_caches(caches):
    return [[(np.asarray(k, np.float64), np.asarray(v, np.float64)) for k, v in per]
            for per in caches]


GOLDEN = Path(__file__).resolve().parent / "golden"


def golden(name):
    """Values a page prints for a worked example, from tests/golden/<name>.txt:
    `key: v1 v2 ...` lines of integers ('#' starts a comment).  A key with one
    value maps to an int, with several to a list."""
    out = {}
    for line in (GOLDEN / f"{name}.txt").read_text(encoding="utf-8").splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, vals = line.split(":", 1)
        nums = [int(v) for v in vals.split()]
        out[key.strip()] = nums[0] if len(nums) == 1 else nums
    return out
