"""Comparison rules shared by the GPU parity tests.

* Indexer scores: relative RMS error sqrt(sum (I_gpu - I_ref)^2 / sum I_ref^2)
  over all valid (row, s) must be <= 1e-3.
* Selections: the GPU set must be a valid top-k set.  Positions whose
  oracle score lies within 1e-3 * |tau| of the oracle's k-th score tau are
  ambiguous (Sec. 5.2 of the analysis page: compare the cutoff, then the
  strictly-above set, then ties); every other position must agree on
  membership.  Rows with n_p <= k must be exactly 0..n_p-1.
* Attention output (bf16): per (row, head), max_d |o_gpu - o_ref| /
  max_d |o_ref| <= 2e-2 against the float64 oracle.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import dsa_oracle as O
from synth import workloads as W

SCORE_REL_RMS = 1e-3
BAND_REL = 1e-3
ATTN_MAX_REL = 2e-2
LSE_ABS = 2e-3


def to_dev(arr: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    return O.bf16_decode(t.cpu().numpy().view(np.uint16))


# ---------------------------------------------------------------- oracle inputs
class HostSide:
    """Oracle-side view of a workload, regenerated on the host from the seed
    (never read back from the GPU)."""

    def __init__(self, wl: W.Workload, b: int = 0):
        self.wl, self.b = wl, b
        self._k = None

    def k_all(self):
        if self._k is None:
            c, s = W.k_idx_fp8(self.wl, self.b, 0, self.wl.n_kv)
            self._k = O.dequant_e4m3(c, s)
        return self._k

    def q_idx(self, i):
        c, s = W.q_idx_fp8(self.wl, self.b, [i])
        return O.dequant_e4m3(c, s)[0]

    def w(self, i):
        return O.bf16_decode(W.w_idx_bf16(self.wl, self.b, [i]))[0]

    def q(self, i):
        return O.bf16_decode(W.q_bf16(self.wl, self.b, [i]))[0]

    def kv_rows(self, rows):
        return O.bf16_decode(W.kv_bf16_rows(self.wl, self.b, rows))

    def scores(self, i):
        return O.indexer_row(self.q_idx(i), self.w(i), self.k_all(), self.wl.q_pos0 + i)

    def attention(self, i, sel):
        """Oracle attention of row i over `sel` (generating only those kv rows)."""
        s = np.asarray(sel)
        s = s[s >= 0]
        kv = self.kv_rows(s) if s.size else np.zeros((0, self.wl.dim_qk))
        return O.sparse_mla_row(self.q(i), kv, np.arange(s.size), self.wl.sm_scale, self.wl.dim_v)


# ---------------------------------------------------------------- checks
def score_rel_rms(pairs):
    num = sum(float(((g.astype(np.float64) - r.astype(np.float64)) ** 2).sum()) for g, r in pairs)
    den = sum(float((r.astype(np.float64) ** 2).sum()) for _, r in pairs)
    return np.sqrt(num / max(den, 1e-300))


def check_selection(gpu_row: np.ndarray, ref_scores: np.ndarray, k: int, rel: float = BAND_REL):
    """Returns (recall R_k vs the oracle set, number of ambiguous positions).
    Raises AssertionError on a violation."""
    n = ref_scores.shape[0]
    m = min(k, n)
    assert gpu_row.shape == (k,)
    chosen = gpu_row[:m]
    assert np.all(gpu_row[m:] == -1), "padding must be -1"
    assert np.all(chosen >= 0) and np.all(chosen < n), "index out of range"
    assert np.all(np.diff(chosen) > 0), "indices must be strictly ascending"
    if n <= k:
        assert np.array_equal(chosen, np.arange(n)), "short row must select everything"
        return 1.0, 0
    ref = O.topk_row(ref_scores, k)[:m]
    x = ref_scores.astype(np.float64)
    tau = np.sort(x)[::-1][m - 1]
    amb = np.abs(x - tau) <= rel * abs(tau)
    in_gpu = np.zeros(n, bool); in_gpu[chosen] = True
    in_ref = np.zeros(n, bool); in_ref[ref] = True
    bad = (in_gpu != in_ref) & ~amb
    assert not np.any(bad), f"membership differs outside the tie band at {np.nonzero(bad)[0][:10]}"
    return float(np.intersect1d(chosen, ref).size) / m, int(amb.sum())


def attn_errors(o_gpu: np.ndarray, o_ref: np.ndarray):
    """Per head: max |diff| / max |ref| (o arrays [H, Dv])."""
    num = np.abs(o_gpu - o_ref).max(axis=1)
    den = np.maximum(np.abs(o_ref).max(axis=1), 1e-30)
    return num / den
