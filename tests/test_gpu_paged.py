"""GPU parity of the paged / variable-length path (dsa_*_paged and
dsa_gather_stats, through the C ABI) against the oracle: every sequence has
its own length, its caches live in a page pool at random places, and its
query rows are its last n_q tokens.  The oracle regenerates each sequence's
logical tokens on the host (the pool is only a permutation of them)."""
import numpy as np
import pytest
import torch

import sparse_attention_long_amd as dsa
from oracle import dsa_oracle as O
from sparse_attention_long_amd import dsa as D
from synth import device as SD
from synth import workloads as W

from dsa_parity import (ATTN_MAX_REL, LSE_ABS, SCORE_REL_RMS, HostSide, attn_errors, bf16_tensor_to_f64,
                        check_selection, score_rel_rms)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()   # raises if the HIP library is missing: no fallback path exists
    yield
    torch.cuda.synchronize()


def _say(*a):
    print(*a, flush=True)


# name -> (workload, page_size, shortest length)
CASES = {
    # decode, production dims; lengths 1000..12000 (some rows shorter than k = 2048); split attention
    "decode_prod_p64": (W.custom("dec64", batch=6, n_kv=12000, q_pos0=11999), 64, 1000),
    "decode_prod_p256": (W.custom("dec64", batch=3, n_kv=9000, q_pos0=8999), 256, 3000),
    # 3 new tokens per sequence (decode form of the indexer, several rows)
    "decode3_prod": (W.custom("dec64", batch=3, n_q=3, n_kv=5000, q_pos0=4997), 64, 2500),
    # prefill chunk of 40 rows per sequence: production and tiny dims
    "prefill_prod": (W.custom("p4k", batch=2, n_q=40, n_kv=2600, q_pos0=2560), 64, 900),
    "prefill_tiny": (W.custom("tiny", batch=3, n_q=40, n_kv=256, q_pos0=216), 64, 40),
}


def _setup(name):
    wl, P, lo = CASES[name]
    lay = W.paged_layout(wl, P, min_len=lo)
    d = SD.fill_paged(wl, lay)
    pk = D.PagedKV.of(d["seq_lens"], d["page_table"], P, lay.max_pages, lay.num_pages)
    return wl, lay, d, pk, D.Dims.of(wl)


def _positions(wl, lay, b):
    return O.varlen_positions(lay.seq_lens[b], wl.n_q)


@pytest.mark.parametrize("name", list(CASES))
def test_paged_indexer_matches_oracle(name):
    wl, lay, d, pk, dims = _setup(name)
    sc = torch.full((wl.batch, wl.n_q, wl.n_kv), float("nan"), dtype=torch.float32, device="cuda")
    D.dsa_indexer_scores_paged(dims, pk, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], sc,
                               wl.n_kv)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    pairs = []
    for b in range(wl.batch):
        hs = HostSide(wl, b)
        k_all = hs.k_all()[:lay.seq_lens[b]]
        for i, p in enumerate(_positions(wl, lay, b)):
            ref = O.indexer_row(hs.q_idx(i), hs.w(i), k_all, p)
            n = ref.shape[0]
            assert n == p + 1
            assert np.all(np.isnan(got[b, i, n:])), (b, i, "written past the row's candidates")
            pairs.append((got[b, i, :n], ref))
    err = score_rel_rms(pairs)
    _say(name, "paged indexer rel RMS", err)
    assert err <= SCORE_REL_RMS


@pytest.mark.parametrize("name", list(CASES))
def test_paged_topk_and_attention_match_oracle(name):
    wl, lay, d, pk, dims = _setup(name)
    k = wl.topk
    # top-k on the oracle's own scores: exact, no band
    sc = np.full((wl.batch, wl.n_q, wl.n_kv), np.nan, np.float32)
    ref_sel = np.full((wl.batch, wl.n_q, k), -1, np.int32)
    hosts = [HostSide(wl, b) for b in range(wl.batch)]
    for b in range(wl.batch):
        k_all = hosts[b].k_all()[:lay.seq_lens[b]]
        for i, p in enumerate(_positions(wl, lay, b)):
            r = O.indexer_row(hosts[b].q_idx(i), hosts[b].w(i), k_all, p)
            sc[b, i, :r.shape[0]] = r
            ref_sel[b, i] = O.topk_row(r, k)
    idx = torch.empty((wl.batch, wl.n_q, k), dtype=torch.int32, device="cuda")
    D.dsa_topk_paged(dims, pk, torch.from_numpy(sc).cuda(), wl.n_kv, idx)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), ref_sel)
    # attention over the oracle's selection
    nws = D.dsa_attn_workspace_size(dims)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.batch, wl.n_q, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.batch, wl.n_q, wl.heads), dtype=torch.float32, device="cuda")
    D.dsa_sparse_mla_attn_paged(dims, pk, d["q"], d["kv"], torch.from_numpy(ref_sel).cuda(), wl.sm_scale, out, lse,
                                ws, nws)
    torch.cuda.synchronize()
    o = bf16_tensor_to_f64(out)
    l = lse.cpu().numpy()
    worst = 0.0
    for b in range(wl.batch):
        for i in range(wl.n_q):
            o_ref, lse_ref = hosts[b].attention(i, ref_sel[b, i])
            worst = max(worst, float(attn_errors(o[b, i], o_ref).max()))
            assert np.abs(l[b, i] - lse_ref).max() <= LSE_ABS, (b, i)
    _say(name, "paged attention worst normwise error", worst)
    assert worst <= ATTN_MAX_REL


@pytest.mark.parametrize("name", ["decode_prod_p64", "decode3_prod", "prefill_prod", "prefill_tiny"])
def test_paged_forward_bitwise_equals_chained_calls(name):
    wl, lay, d, pk, dims = _setup(name)
    k = wl.topk
    out = torch.empty((wl.batch, wl.n_q, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.batch, wl.n_q, wl.heads), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.batch, wl.n_q, k), dtype=torch.int32, device="cuda")
    fws = D.dsa_forward_workspace_size(dims)
    ws = torch.empty(fws, dtype=torch.uint8, device="cuda")
    D.dsa_forward_paged(dims, pk, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], d["q"], d["kv"],
                        wl.sm_scale, out, lse, idx, ws, fws)
    sc = torch.empty((wl.batch, wl.n_q, wl.n_kv), dtype=torch.float32, device="cuda")
    D.dsa_indexer_scores_paged(dims, pk, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], sc,
                               wl.n_kv)
    idx_c = torch.empty_like(idx)
    D.dsa_topk_paged(dims, pk, sc, wl.n_kv, idx_c)
    nws = D.dsa_attn_workspace_size(dims)
    aws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    out_c = torch.empty_like(out)
    lse_c = torch.empty_like(lse)
    D.dsa_sparse_mla_attn_paged(dims, pk, d["q"], d["kv"], idx_c, wl.sm_scale, out_c, lse_c, aws, nws)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_c)
    assert torch.equal(out, out_c)
    assert torch.equal(lse.view(torch.int32), lse_c.view(torch.int32))
    # the selection itself obeys the band rule against the oracle
    got = idx.cpu().numpy()
    for b in range(wl.batch):
        hs = HostSide(wl, b)
        k_all = hs.k_all()[:lay.seq_lens[b]]
        for i, p in enumerate(_positions(wl, lay, b)):
            check_selection(got[b, i], O.indexer_row(hs.q_idx(i), hs.w(i), k_all, p), k)


@pytest.mark.parametrize("name", ["decode_prod_p64", "prefill_prod", "prefill_tiny"])
def test_full_length_paged_equals_dense_bitwise(name):
    # Every sequence at n_kv with its pages shuffled: the paged calls see the
    # same tokens as the dense calls and must return the same bits.
    wl, P, _ = CASES[name]
    assert wl.q_pos0 == wl.n_kv - wl.n_q   # the dense calls' positions equal the full-length ones
    lay = W.paged_layout(wl, P, full=True)
    dp = SD.fill_paged(wl, lay)
    dd = SD.fill_inputs(wl)
    pk = D.PagedKV.of(dp["seq_lens"], dp["page_table"], P, lay.max_pages, lay.num_pages)
    dims = D.Dims.of(wl)
    k = wl.topk
    res = []
    for paged in (True, False):
        d = dp if paged else dd
        out = torch.empty((wl.batch, wl.n_q, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
        lse = torch.empty((wl.batch, wl.n_q, wl.heads), dtype=torch.float32, device="cuda")
        idx = torch.empty((wl.batch, wl.n_q, k), dtype=torch.int32, device="cuda")
        sc = torch.full((wl.batch, wl.n_q, wl.n_kv), float("nan"), dtype=torch.float32, device="cuda")
        fws = D.dsa_forward_workspace_size(dims)
        ws = torch.empty(fws, dtype=torch.uint8, device="cuda")
        args = (d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"])
        if paged:
            D.dsa_indexer_scores_paged(dims, pk, *args, sc, wl.n_kv)
            D.dsa_forward_paged(dims, pk, *args, d["q"], d["kv"], wl.sm_scale, out, lse, idx, ws, fws)
        else:
            D.dsa_indexer_scores(dims, *args, sc, wl.n_kv)
            D.dsa_forward(dims, *args, d["q"], d["kv"], wl.sm_scale, out, lse, idx, ws, fws)
        torch.cuda.synchronize()
        res.append((sc.cpu(), idx.cpu(), out.cpu(), lse.cpu()))
    (s1, i1, o1, l1), (s2, i2, o2, l2) = res
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(i1, i2) and torch.equal(o1, o2) and torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_gather_stats_match_oracle():
    rs = np.random.RandomState(41)
    B, T, k = 3, 7, 2048
    rows = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for i in range(T):
            n = int(rs.randint(1, 200000))
            m = int(rs.randint(0, min(n, k) + 1))
            kind = (b * T + i) % 3
            if kind == 0:
                sel = np.sort(rs.choice(n, m, replace=False))
            elif kind == 1:
                s0 = int(rs.randint(0, max(1, n - m)))
                sel = np.arange(s0, s0 + m)
            else:
                c = np.sort(rs.choice(n, max(1, m // 16), replace=False))
                sel = np.unique(np.concatenate([c + j for j in range(16)]))[:m]
            rows[b, i, :len(sel)] = sel
    rows[0, 0] = -1                                   # an empty row
    for ps in (1, 64, 4096):
        stats = torch.full((B, T, 3), -7, dtype=torch.int32, device="cuda")
        dims = D.Dims(batch=B, n_q=T, n_kv=200000, q_pos0=0, idx_heads=64, idx_dim=128, heads=128, dim_qk=576,
                      dim_v=512, topk=k)
        D.dsa_gather_stats(dims, ps, torch.from_numpy(rows).cuda(), stats)
        torch.cuda.synchronize()
        got = stats.cpu().numpy()
        for b in range(B):
            for i in range(T):
                assert tuple(got[b, i]) == O.gather_stats(rows[b, i], ps), (ps, b, i)


def test_out_of_range_lengths_and_pages_are_clamped():
    # A length above n_kv acts as n_kv and one below n_q as n_q; a page entry
    # past the pool acts as the last page.  Nothing may fault, and the results
    # equal those of the clamped layout.
    wl, P, lo = CASES["decode_prod_p64"]
    lay = W.paged_layout(wl, P, min_len=lo)
    d = SD.fill_paged(wl, lay)
    bad_lens = list(lay.seq_lens)
    bad_lens[0], bad_lens[1] = wl.n_kv + 500, -3
    good_lens = list(bad_lens)
    good_lens[0], good_lens[1] = wl.n_kv, wl.n_q
    bad_table = lay.table.copy()
    bad_table[2, 3] = lay.num_pages + 11
    good_table = bad_table.copy()
    good_table[2, 3] = lay.num_pages - 1
    outs = []
    for lens, table in ((bad_lens, bad_table), (good_lens, good_table)):
        sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        pt = torch.from_numpy(table).cuda()
        pk = D.PagedKV.of(sl, pt, P, lay.max_pages, lay.num_pages)
        dims = D.Dims.of(wl)
        out = torch.empty((wl.batch, wl.n_q, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
        idx = torch.empty((wl.batch, wl.n_q, wl.topk), dtype=torch.int32, device="cuda")
        fws = D.dsa_forward_workspace_size(dims)
        ws = torch.empty(fws, dtype=torch.uint8, device="cuda")
        D.dsa_forward_paged(dims, pk, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], d["q"],
                            d["kv"], wl.sm_scale, out, None, idx, ws, fws)
        torch.cuda.synchronize()
        outs.append((idx.cpu(), out.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
