"""GPU parity of the forward indexer KL on the selected set (dsa_indexer_kl,
dsa_forward_kl through the C ABI) against the oracle.

Tolerance.  Given the same index scores and selection, the GPU recomputes
the attention weights from bf16 q and c with fp32 accumulation and fp32
exp/log; their relative error is ~1e-6, and the KL moves by about that much
times (1 + |ln p - ln q|).  The test allows |KL_gpu - KL_ref| <= 1e-3 *
(1 + |KL_ref|).  End to end the GPU's own index scores differ from the
oracle's; the KL of Eq. (4) changes by at most 2 * max_s |dI_s| when the
scores move by dI (its gradient in I is q - p, whose L1 norm is <= 2), so
that bound is added there."""
import numpy as np
import pytest
import torch

import sparse_attention_long_amd as dsa
from oracle import dsa_oracle as O
from sparse_attention_long_amd import dsa as D
from synth import device as SD
from synth import workloads as W

from dsa_parity import HostSide, check_selection

pytestmark = pytest.mark.gpu

KL_REL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()   # raises if the HIP library is missing: no fallback path exists
    yield
    torch.cuda.synchronize()


def _say(*a):
    print(*a, flush=True)


CASES = {
    # prefill rows deep in a 4K sequence (full 2048-token selections)
    "prefill_prod": W.custom("p4k", n_q=12, q_pos0=4096 - 12),
    # rows near the start (selection = every candidate, some rows short)
    "prefill_head": W.custom("p4k", n_q=20, q_pos0=2040),
    # decode rows of several sequences
    "decode_prod": W.custom("dec64", batch=4, n_kv=6000, q_pos0=5999),
    # tiny dims, all rows
    "tiny": W.WORKLOADS["tiny"],
}


def _oracle_rows(wl, hosts, positions_of):
    """Oracle scores [B,T,S] (NaN past a row), selections [B,T,k]."""
    sc = np.full((wl.batch, wl.n_q, wl.n_kv), np.nan, np.float32)
    sel = np.full((wl.batch, wl.n_q, wl.topk), -1, np.int32)
    for b in range(wl.batch):
        k_all = hosts[b].k_all()
        for i, (p, n_kv) in enumerate(positions_of(b)):
            r = O.indexer_row(hosts[b].q_idx(i), hosts[b].w(i), k_all[:n_kv], p)
            sc[b, i, :r.shape[0]] = r
            sel[b, i] = O.topk_row(r, wl.topk)
    return sc, sel


def _kl_ref(wl, host, i, sel_row, sc_row):
    s = np.asarray(sel_row)
    s = s[s >= 0]
    kv = host.kv_rows(s) if s.size else np.zeros((0, wl.dim_qk))
    # the oracle works on the gathered rows: remap the selection to 0..m-1
    return O.indexer_kl_row(host.q(i), kv, np.arange(s.size), sc_row[s].astype(np.float64), wl.sm_scale, wl.dim_v)


@pytest.mark.parametrize("name", list(CASES))
def test_indexer_kl_matches_oracle(name):
    wl = CASES[name]
    d = SD.fill_inputs(wl)
    dims = D.Dims.of(wl)
    hosts = [HostSide(wl, b) for b in range(wl.batch)]
    sc, sel = _oracle_rows(wl, hosts, lambda b: [(wl.q_pos0 + i, wl.n_kv) for i in range(wl.n_q)])
    idx = torch.from_numpy(sel).cuda()
    out = torch.empty((wl.batch, wl.n_q, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.batch, wl.n_q, wl.heads), dtype=torch.float32, device="cuda")
    nws = D.dsa_attn_workspace_size(dims)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    D.dsa_sparse_mla_attn(dims, d["q"], d["kv"], idx, wl.sm_scale, out, lse, ws, nws)
    kl = torch.full((wl.batch, wl.n_q), float("nan"), dtype=torch.float32, device="cuda")
    D.dsa_indexer_kl(dims, None, d["q"], d["kv"], idx, lse, torch.from_numpy(sc).cuda(), wl.n_kv, wl.sm_scale, kl)
    torch.cuda.synchronize()
    got = kl.cpu().numpy()
    worst = 0.0
    for b in range(wl.batch):
        for i in range(wl.n_q):
            ref = _kl_ref(wl, hosts[b], i, sel[b, i], sc[b, i])
            err = abs(float(got[b, i]) - ref)
            worst = max(worst, err / (1 + abs(ref)))
            assert err <= KL_REL * (1 + abs(ref)), (b, i, float(got[b, i]), ref)
    _say(name, "indexer KL worst relative error", worst, "sample", float(got[0, 0]))


def test_indexer_kl_paged_matches_oracle():
    wl = W.custom("dec64", batch=5, n_kv=7000, q_pos0=6999)
    P = 64
    lay = W.paged_layout(wl, P, min_len=1500)
    d = SD.fill_paged(wl, lay)
    pk = D.PagedKV.of(d["seq_lens"], d["page_table"], P, lay.max_pages, lay.num_pages)
    dims = D.Dims.of(wl)
    hosts = [HostSide(wl, b) for b in range(wl.batch)]
    sc, sel = _oracle_rows(wl, hosts, lambda b: [(lay.seq_lens[b] - 1, lay.seq_lens[b])])
    idx = torch.from_numpy(sel).cuda()
    out = torch.empty((wl.batch, 1, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.batch, 1, wl.heads), dtype=torch.float32, device="cuda")
    nws = D.dsa_attn_workspace_size(dims)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    D.dsa_sparse_mla_attn_paged(dims, pk, d["q"], d["kv"], idx, wl.sm_scale, out, lse, ws, nws)
    kl = torch.empty((wl.batch, 1), dtype=torch.float32, device="cuda")
    D.dsa_indexer_kl(dims, pk, d["q"], d["kv"], idx, lse, torch.from_numpy(sc).cuda(), wl.n_kv, wl.sm_scale, kl)
    torch.cuda.synchronize()
    got = kl.cpu().numpy()
    for b in range(wl.batch):
        ref = _kl_ref(wl, hosts[b], 0, sel[b, 0], sc[b, 0])
        assert abs(float(got[b, 0]) - ref) <= KL_REL * (1 + abs(ref)), (b, float(got[b, 0]), ref)


@pytest.mark.parametrize("name", ["prefill_prod", "decode_prod", "tiny"])
def test_forward_kl_bitwise_and_end_to_end(name):
    wl = CASES[name]
    d = SD.fill_inputs(wl)
    dims = D.Dims.of(wl)
    B, T, k = wl.batch, wl.n_q, wl.topk
    out = torch.empty((B, T, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    lse = torch.empty((B, T, wl.heads), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, T, k), dtype=torch.int32, device="cuda")
    kl = torch.empty((B, T), dtype=torch.float32, device="cuda")
    fws = D.dsa_forward_workspace_size(dims)
    ws = torch.empty(fws, dtype=torch.uint8, device="cuda")
    args = (d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"])
    D.dsa_forward_kl(dims, None, *args, d["q"], d["kv"], wl.sm_scale, out, lse, idx, kl, ws, fws)
    # chained: indexer -> top-k -> attention -> KL
    sc = torch.empty((B, T, wl.n_kv), dtype=torch.float32, device="cuda")
    D.dsa_indexer_scores(dims, *args, sc, wl.n_kv)
    idx_c = torch.empty_like(idx)
    D.dsa_topk(dims, sc, wl.n_kv, idx_c)
    nws = D.dsa_attn_workspace_size(dims)
    aws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    out_c, lse_c, kl_c = torch.empty_like(out), torch.empty_like(lse), torch.empty_like(kl)
    D.dsa_sparse_mla_attn(dims, d["q"], d["kv"], idx_c, wl.sm_scale, out_c, lse_c, aws, nws)
    D.dsa_indexer_kl(dims, None, d["q"], d["kv"], idx_c, lse_c, sc, wl.n_kv, wl.sm_scale, kl_c)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_c) and torch.equal(out, out_c)
    assert torch.equal(kl.view(torch.int32), kl_c.view(torch.int32))
    # end to end against the oracle on the GPU's (band-checked) selection
    got_kl, got_idx, got_sc = kl.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    for b in range(B):
        hs = HostSide(wl, b)
        for i in range(T):
            ref_sc = hs.scores(i)
            check_selection(got_idx[b, i], ref_sc, k)
            s = got_idx[b, i][got_idx[b, i] >= 0]
            ref = O.indexer_kl_row(hs.q(i), hs.kv_rows(s), np.arange(s.size), ref_sc[s].astype(np.float64),
                                   wl.sm_scale, wl.dim_v)
            d_i = float(np.abs(got_sc[b, i, s].astype(np.float64) - ref_sc[s]).max())
            assert abs(float(got_kl[b, i]) - ref) <= 2 * d_i + KL_REL * (1 + abs(ref)), (b, i, got_kl[b, i], ref, d_i)
