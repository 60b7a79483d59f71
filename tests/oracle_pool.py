"""Oracle rows of full-size workloads, evaluated in parallel worker processes.

Test infrastructure for the full-size parity checks.  The workers import only
numpy, the oracle and the seeded input generators: never torch and never the
GPU library.  They start with the "spawn" method (fresh interpreters, nothing
inherited from a process that holds the GPU) and use one BLAS thread each.

Every expected value comes from the oracle on inputs regenerated on the host
from the workload's seed.  The GPU's results enter only as the values under
test: its selection (checked against the oracle scores with the band rule
before the oracle attends over it) and its output and log-sum-exp rows.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

from oracle import dsa_oracle as O
from synth import workloads as W

BAND_REL = 1e-3      # selection band: |I_ref(s) - tau| <= 1e-3 |tau| is ambiguous
ELEM_FLOOR = 1e-3    # elementwise relative error floor, as a fraction of the row's max |o_ref|

_cache = {}


def _init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _k_all(wl, b):
    key = (wl, b)
    if key not in _cache:
        _cache.clear()
        c, s = W.k_idx_fp8(wl, b, 0, wl.n_kv)
        _cache[key] = O.dequant_e4m3(c, s)
    return _cache[key]


def selection_check(gsel, ref_scores, k):
    """(ok, message, recall, ambiguous count, cutoff margin) of a GPU selection
    row against the oracle scores: a valid top-k set, agreeing with the
    oracle's set at every position outside the tie band; rows with n_p <= k
    must select everything.  The margin is the oracle's s_(m) - s_(m+1)
    (Sec. 5.2, Eq. (18)), or None for a row that selects everything."""
    n = ref_scores.shape[0]
    m = min(k, n)
    chosen = gsel[:m]
    if not np.all(gsel[m:] == -1):
        return False, "padding must be -1", 0.0, 0, None
    if not (np.all(chosen >= 0) and np.all(chosen < n)):
        return False, "index out of range", 0.0, 0, None
    if not np.all(np.diff(chosen) > 0):
        return False, "indices must be strictly ascending", 0.0, 0, None
    if n <= k:
        ok = np.array_equal(chosen, np.arange(n))
        return ok, "" if ok else "short row must select everything", 1.0, 0, None
    ref = O.topk_row(ref_scores, k)[:m]
    x = ref_scores.astype(np.float64)
    srt = np.sort(x)[::-1]
    tau = srt[m - 1]
    amb = np.abs(x - tau) <= BAND_REL * abs(tau)
    in_gpu = np.zeros(n, bool)
    in_gpu[chosen] = True
    in_ref = np.zeros(n, bool)
    in_ref[ref] = True
    bad = (in_gpu != in_ref) & ~amb
    if np.any(bad):
        return False, f"membership differs outside the tie band at {np.nonzero(bad)[0][:10]}", 0.0, int(amb.sum()), None
    recall = float(np.intersect1d(chosen, ref).size) / m
    return True, "", recall, int(amb.sum()), float(srt[m - 1] - srt[m])


def _rows_task(args):
    """Rows of sequence b: oracle scores, the selection check of the GPU's row,
    and the oracle attention over the GPU's selection compared with the GPU's
    output and lse.  Returns one dict per row."""
    wl, b, rows, gsel, gout_bits, glse = args
    k_all = _k_all(wl, b)
    res = []
    for n_, i in enumerate(rows):
        p = wl.q_pos0 + i
        qc, qs = W.q_idx_fp8(wl, b, [i])
        qi = O.dequant_e4m3(qc, qs)[0]
        w = O.bf16_decode(W.w_idx_bf16(wl, b, [i]))[0]
        ref_sc = O.indexer_row(qi, w, k_all, p)
        ok, msg, recall, amb, margin = selection_check(gsel[n_], ref_sc, wl.topk)
        r = {"b": b, "i": i, "ok": ok, "msg": msg, "recall": recall, "amb": amb, "margin": margin}
        if ok:
            sel = gsel[n_][gsel[n_] >= 0]
            kv = O.bf16_decode(W.kv_bf16_rows(wl, b, sel))
            q = O.bf16_decode(W.q_bf16(wl, b, [i]))[0]
            ref_o, ref_lse = O.sparse_mla_row(q, kv, np.arange(sel.size), wl.sm_scale, wl.dim_v)
            o = O.bf16_decode(gout_bits[n_])
            diff = np.abs(o - ref_o)
            rowmax = np.abs(ref_o).max(axis=1)
            r["normwise"] = float((diff.max(axis=1) / np.maximum(rowmax, 1e-30)).max())
            r["elementwise"] = float((diff / np.maximum(np.abs(ref_o), ELEM_FLOOR * rowmax[:, None])).max())
            r["lse"] = float(np.abs(glse[n_] - ref_lse).max())
        res.append(r)
    return res


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def check_rows(wl, rows_by_seq, idx, out_bits, lse, rows_per_task=16):
    """Evaluate the oracle for rows_by_seq {b: [i, ...]} against the GPU's
    results in a spawned pool.  idx, out_bits and lse are either whole
    arrays ([B, T, k] int32, [B, T, H, Dv] bf16 bits, [B, T, H]) or dicts
    {b: array} holding only the listed rows of sequence b, in list order.
    Returns the per-row dicts in order."""
    def rows_of(x, b, pos, rr):
        return x[b][pos] if isinstance(x, dict) else x[b, rr]

    tasks = []
    for b, rows in rows_by_seq.items():
        rows = list(rows)
        for j in range(0, len(rows), rows_per_task):
            rr = rows[j:j + rows_per_task]
            pos = list(range(j, j + len(rr)))
            tasks.append((wl, b, rr, rows_of(idx, b, pos, rr), rows_of(out_bits, b, pos, rr),
                          rows_of(lse, b, pos, rr)))
    ctx = mp.get_context("spawn")
    with ctx.Pool(min(workers(), len(tasks)), initializer=_init) as pool:
        parts = pool.map(_rows_task, tasks, chunksize=1)
    return [r for part in parts for r in part]


def summarise(results):
    """Aggregate of per-row dicts: rows checked, rows compared, worst errors,
    mean recall R_k (Sec. 5, Eq. (14)), ambiguous positions, and the cutoff
    margin distribution (Sec. 5.2, Eq. (18)) as quantiles and a log10
    histogram."""
    cmp = [r for r in results if "normwise" in r]
    margins = np.array([r["margin"] for r in results if r["margin"] is not None])
    s = {"rows": len(results), "compared": len(cmp),
         "failed": [(r["b"], r["i"], r["msg"]) for r in results if not r["ok"]],
         "normwise_max": max((r["normwise"] for r in cmp), default=0.0),
         "elementwise_max": max((r["elementwise"] for r in cmp), default=0.0),
         "lse_max": max((r["lse"] for r in cmp), default=0.0),
         "recall_mean": float(np.mean([r["recall"] for r in results])) if results else 0.0,
         "ambiguous": int(sum(r["amb"] for r in results))}
    if margins.size:
        s["margin_quantiles"] = {q: float(np.quantile(margins, q)) for q in (0.0, 0.01, 0.5, 0.99, 1.0)}
        edges = [-np.inf, 1e-7, 1e-6, 1e-5, 1e-4, 1e-3, 1e-2, 1e-1, np.inf]
        s["margin_hist_log10"] = {f"<{e:g}": int(c) for e, c in zip(edges[1:], np.histogram(margins, edges)[0])}
    return s
