"""The parallel oracle-row checker used by the full-size GPU parity tests,
run on the CPU: results made by the oracle itself pass with bf16-sized
errors, and a selection that disagrees outside the tie band, or an output
off by more than the tolerance, is reported."""
import numpy as np

import oracle_pool
from oracle import dsa_oracle as O
from synth import gen
from synth import workloads as W


def _oracle_results(wl, rows):
    B, k = wl.batch, wl.topk
    idx = np.full((B, wl.n_q, k), -1, np.int32)
    out = np.zeros((B, wl.n_q, wl.heads, wl.dim_v), np.uint16)
    lse = np.zeros((B, wl.n_q, wl.heads), np.float32)
    for b, rr in rows.items():
        c, s = W.k_idx_fp8(wl, b, 0, wl.n_kv)
        k_all = O.dequant_e4m3(c, s)
        kv = O.bf16_decode(W.kv_bf16_rows(wl, b, np.arange(wl.n_kv)))
        for i in rr:
            qc, qs = W.q_idx_fp8(wl, b, [i])
            sc = O.indexer_row(O.dequant_e4m3(qc, qs)[0], O.bf16_decode(W.w_idx_bf16(wl, b, [i]))[0], k_all,
                               wl.q_pos0 + i)
            sel = O.topk_row(sc, k)
            o, l = O.sparse_mla_row(O.bf16_decode(W.q_bf16(wl, b, [i]))[0], kv, sel, wl.sm_scale, wl.dim_v)
            idx[b, i], out[b, i], lse[b, i] = sel, gen.f32_to_bf16_bits(o.astype(np.float32)), l
    return idx, out, lse


def test_pool_accepts_oracle_results_and_reports_mistakes():
    wl = W.custom("tiny", batch=2)
    rows = {0: [0, 5, 40, 128, 255], 1: [1, 31, 32, 200]}
    idx, out, lse = _oracle_results(wl, rows)
    s = oracle_pool.summarise(oracle_pool.check_rows(wl, rows, idx, out, lse, rows_per_task=2))
    assert not s["failed"] and s["compared"] == s["rows"] == 9
    assert s["normwise_max"] <= 2 ** -8 and s["lse_max"] <= 1e-5 and s["recall_mean"] == 1.0
    assert sum(s["margin_hist_log10"].values()) == 5      # rows with n_p <= k = 32 have no cutoff
    # a selection that swaps the row's best key for one far below the cutoff
    bad = idx.copy()
    sel = idx[1, 200].copy()
    c, s_ = W.k_idx_fp8(wl, 1, 0, wl.n_kv)
    qc, qs = W.q_idx_fp8(wl, 1, [200])
    sc = O.indexer_row(O.dequant_e4m3(qc, qs)[0], O.bf16_decode(W.w_idx_bf16(wl, 1, [200]))[0],
                       O.dequant_e4m3(c, s_), 200)
    worst_out = int(np.argsort(sc, kind="stable")[0])     # the lowest score: far outside the band
    best_in = int(sel[np.argmax(sc[sel])])
    bad[1, 200] = np.sort(np.where(sel == best_in, worst_out, sel))
    res = oracle_pool.check_rows(wl, {1: [200]}, bad, out, lse)
    assert not res[0]["ok"] and "tie band" in res[0]["msg"]
    # an output row off by 5% in one head
    o2 = out.copy()
    o2[0, 128, 3] = gen.f32_to_bf16_bits((O.bf16_decode(out[0, 128, 3]) * 1.05).astype(np.float32))
    r = oracle_pool.check_rows(wl, {0: [128]}, idx, o2, lse)[0]
    assert r["ok"] and r["normwise"] > 2e-2
