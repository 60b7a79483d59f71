"""GPU parity of the masked MHA-mode short-prefill path (dsa_selection_mask,
dsa_mha_decompress, dsa_masked_mha_attn, dsa_masked_mha_forward through the
C ABI) against the oracle.

Tolerances.
* Selection bitmap: bit-exact.
* Decompressed keys/values: the GPU rounds an fp32 sum once to bf16, so
  |gpu - ref| <= 2^-8 |ref| + 1e-6 * sum_c |W c| per element.
* Attention: per (row, head) max |o_gpu - o_ref| / max |o_ref| <= 2e-2.
  The per-head keys the GPU attends with are bf16 (relative rounding
  <= 2^-9 per element), so each logit may move by up to
  e_z = sm_scale * 2^-9 * sum_d |q_d k_d|; the lse is compared with
  |dlse| <= 2e-3 + 2 * max_s e_z(s) (the log-sum-exp moves by at most the
  largest logit change)."""
import numpy as np
import pytest
import torch

import sparse_attention_long_amd as dsa
from oracle import dsa_oracle as O
from sparse_attention_long_amd import dsa as D
from synth import device as SD
from synth import workloads as W

from dsa_parity import ATTN_MAX_REL, LSE_ABS, HostSide, attn_errors, bf16_tensor_to_f64, check_selection

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


CASES = {
    # small dims (dn 32, rope 16, dvh 32), 256 rows, k = 32: real masks from row 32 on
    "tiny": W.WORKLOADS["tiny"],
    # 200 ragged rows from position 0: every causal key selected (dense causal)
    "p4k_head": W.custom("p4k", n_q=200, n_kv=200, heads=16),
    # rows deep in a 3K context: 2048 of ~3000 keys selected
    "p4k_deep": W.custom("p4k", n_q=160, n_kv=3060, q_pos0=2900, heads=16),
    # two sequences, a few keys masked per row
    "batch2": W.custom("p4k", batch=2, n_q=96, n_kv=2196, q_pos0=2100, heads=8),
    # sparse selections (64 of ~600 keys): most chunks hold no selected key
    "small_k": W.custom("p4k", n_q=130, n_kv=700, q_pos0=570, topk=64, heads=8),
    # small dims, three sequences, 77 ragged rows continuing a prefill at position 179
    "tiny_b3": W.custom("tiny", batch=3, n_q=77, q_pos0=179),
}


class MhaHost:
    """Oracle-side MHA inputs of a workload (regenerated from the seed)."""

    def __init__(self, wl):
        self.wl = wl
        self.dn, self.dr, self.dvh = W.mha_dims(wl)
        self.w_uk = O.bf16_decode(W.w_mha_bf16(wl, "w_uk"))
        self.w_uv = O.bf16_decode(W.w_mha_bf16(wl, "w_uv"))
        self.hosts = [HostSide(wl, b) for b in range(wl.batch)]
        self._kvh = {}

    def q_mha(self, b, i):
        return O.bf16_decode(W.q_mha_bf16(self.wl, b, [i]))[0]

    def kv(self, b, n):
        return self.hosts[b].kv_rows(np.arange(n))

    def _cached(self, b, n):
        """(latent rows, their decompression) of sequence b, at least n rows."""
        if b not in self._kvh or self._kvh[b][0].shape[0] < n:
            kv = self.kv(b, n)
            self._kvh[b] = (kv, O.mha_decompress(kv, self.w_uk, self.w_uv, self.wl.dim_v))
        return self._kvh[b]

    def kvh(self, b, n):
        return self._cached(b, n)[1]

    def row(self, b, i, sel):
        wl = self.wl
        p = wl.q_pos0 + i
        n = min(p + 1, wl.n_kv)
        kv, kvh = self._cached(b, n)
        return O.masked_mha_row(self.q_mha(b, i), kv[:n], self.w_uk, self.w_uv, sel, p, wl.sm_scale, wl.dim_v,
                                kvh=kvh)

    def logit_err(self, b, i, sel):
        """Largest logit change bf16 keys can cause: sm_scale * 2^-9 * sum |q k| (per head)."""
        wl = self.wl
        p = wl.q_pos0 + i
        n = min(p + 1, wl.n_kv)
        kn, _, _ = self.kvh(b, n)
        s = np.asarray(sel)
        s = s[(s >= 0) & (s < n)]
        if s.size == 0:
            return np.zeros(wl.heads)
        q = self.q_mha(b, i)
        e = np.einsum("hd,hsd->hs", np.abs(q[:, :self.dn]), np.abs(kn[:, s]))
        return wl.sm_scale * 2.0 ** -9 * e.max(axis=1)


def _oracle_selection(wl, mh):
    sel = np.full((wl.batch, wl.n_q, wl.topk), -1, np.int32)
    for b in range(wl.batch):
        for i in range(wl.n_q):
            sel[b, i] = O.topk_row(mh.hosts[b].scores(i), wl.topk)
    return sel


def _check_rows(wl, mh, out, lse, sel, rows, tag):
    worst, worst_lse = 0.0, 0.0
    for b in range(wl.batch):
        for i in rows:
            o_ref, l_ref = mh.row(b, i, sel[b, i])
            err = attn_errors(out[b, i], o_ref)
            assert np.all(err <= ATTN_MAX_REL), (tag, b, i, float(err.max()))
            fin = np.isfinite(l_ref)
            assert np.array_equal(fin, np.isfinite(lse[b, i])), (tag, b, i)
            dl = np.abs(lse[b, i][fin] - l_ref[fin])
            bound = LSE_ABS + 2 * mh.logit_err(b, i, sel[b, i])[fin]
            assert np.all(dl <= bound), (tag, b, i, float(dl.max()))
            worst = max(worst, float(err.max()))
            worst_lse = max(worst_lse, float(dl.max()) if dl.size else 0.0)
    _say(tag, "max rel err", worst, "max |dlse|", worst_lse)


def _alloc_mha(wl, rows_h=None):
    dn, _, dvh = W.mha_dims(wl)
    S = wl.n_kv if rows_h is None else rows_h
    k_mha = torch.full((wl.batch, wl.heads, S, dn), 0x7FC0, dtype=torch.int16, device="cuda")   # NaN fill
    v_mha = torch.full((wl.batch, wl.heads, S, dvh), 0x7FC0, dtype=torch.int16, device="cuda")
    return k_mha, v_mha


@pytest.mark.parametrize("name", list(CASES))
def test_selection_mask_bit_exact(name):
    wl = CASES[name]
    rs = np.random.RandomState(11)
    B, T, S, k = wl.batch, wl.n_q, wl.n_kv, wl.topk
    # arbitrary lists: duplicates, padding, future and out-of-range entries
    idx = rs.randint(-3, S + 5, size=(B, T, k)).astype(np.int32)
    mask = torch.full((B, (S + 31) // 32, T), 0xA5A5A5A5 - (1 << 32), dtype=torch.int32, device="cuda")
    D.dsa_selection_mask(D.Dims.of(wl), torch.from_numpy(idx).cuda(), mask)
    got = mask.cpu().numpy().view(np.uint32)
    for b in range(B):
        for i in range(T):
            bits = O.selection_mask(idx[b, i][idx[b, i] <= wl.q_pos0 + i], S)
            words = np.zeros((S + 31) // 32 * 32, bool)
            words[:S] = bits
            ref = np.packbits(words.reshape(-1, 32)[:, ::-1], axis=1).view(">u4").reshape(-1)
            assert np.array_equal(got[b, :, i], ref.astype(np.uint32)), (b, i)


@pytest.mark.parametrize("name", ["tiny", "p4k_deep"])
def test_decompress_matches_oracle(name):
    wl = CASES[name]
    mh = MhaHost(wl)
    d = SD.fill_inputs(wl)
    m = SD.fill_mha(wl)
    n_rows = wl.n_kv - 37      # a ragged tail; rows past it stay untouched
    k_mha, v_mha = _alloc_mha(wl)
    D.dsa_mha_decompress(D.Dims.of(wl), mh.dn, mh.dvh, d["kv"], m["w_uk"], m["w_uv"], n_rows, k_mha, v_mha)
    torch.cuda.synchronize()
    for b in range(wl.batch):
        c = mh.kv(b, n_rows)[:, :wl.dim_v]
        kn_ref, v_ref, _ = O.mha_decompress(mh.kv(b, n_rows), mh.w_uk, mh.w_uv, wl.dim_v)
        for got_t, ref, w in ((k_mha, kn_ref, mh.w_uk), (v_mha, v_ref, mh.w_uv)):
            got = bf16_tensor_to_f64(got_t[b, :, :n_rows])
            mag = np.matmul(np.abs(c)[None], np.abs(w).transpose(0, 2, 1))
            assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * mag)
            assert np.all(got_t[b, :, n_rows:].cpu().numpy() == 0x7FC0)


@pytest.mark.parametrize("name", list(CASES))
def test_masked_mha_attn_matches_oracle(name):
    wl = CASES[name]
    mh = MhaHost(wl)
    d = SD.fill_inputs(wl)
    m = SD.fill_mha(wl)
    dims = D.Dims.of(wl)
    sel = _oracle_selection(wl, mh)
    mask = torch.empty((wl.batch, (wl.n_kv + 31) // 32, wl.n_q), dtype=torch.int32, device="cuda")
    D.dsa_selection_mask(dims, torch.from_numpy(sel).cuda(), mask)
    k_mha, v_mha = _alloc_mha(wl)
    D.dsa_mha_decompress(dims, mh.dn, mh.dvh, d["kv"], m["w_uk"], m["w_uv"], wl.q_pos0 + wl.n_q, k_mha, v_mha)
    out = torch.empty((wl.batch, wl.n_q, wl.heads, mh.dvh), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.batch, wl.n_q, wl.heads), dtype=torch.float32, device="cuda")
    D.dsa_masked_mha_attn(dims, mh.dn, mh.dvh, m["q_mha"], d["kv"], k_mha, v_mha, mask, wl.sm_scale, out, lse)
    torch.cuda.synchronize()
    o = bf16_tensor_to_f64(out)
    l = lse.cpu().numpy().astype(np.float64)
    rows = range(wl.n_q) if wl.n_q * wl.batch <= 260 else sorted(set(range(0, wl.n_q, 7)) | {wl.n_q - 1})
    _check_rows(wl, mh, o, l, sel, rows, name)


def test_masked_mha_dense_and_empty_masks():
    wl = CASES["p4k_deep"]
    mh = MhaHost(wl)
    d = SD.fill_inputs(wl)
    m = SD.fill_mha(wl)
    dims = D.Dims.of(wl)
    k_mha, v_mha = _alloc_mha(wl)
    D.dsa_mha_decompress(dims, mh.dn, mh.dvh, d["kv"], m["w_uk"], m["w_uv"], wl.q_pos0 + wl.n_q, k_mha, v_mha)
    nc = (wl.n_kv + 31) // 32
    out = torch.empty((1, wl.n_q, wl.heads, mh.dvh), dtype=torch.int16, device="cuda")
    lse = torch.empty((1, wl.n_q, wl.heads), dtype=torch.float32, device="cuda")
    # all bits set: the causal limit alone applies (dense causal MHA attention)
    ones = torch.full((1, nc, wl.n_q), -1, dtype=torch.int32, device="cuda")
    D.dsa_masked_mha_attn(dims, mh.dn, mh.dvh, m["q_mha"], d["kv"], k_mha, v_mha, ones, wl.sm_scale, out, lse)
    torch.cuda.synchronize()
    allsel = np.stack([np.arange(wl.n_kv, dtype=np.int32)] * wl.n_q)[None]
    _check_rows(wl, mh, bf16_tensor_to_f64(out), lse.cpu().numpy().astype(np.float64), allsel,
                [0, 1, 63, 64, 100, wl.n_q - 1], "dense")
    # no bits: out = 0, lse = -inf
    zeros = torch.zeros((1, nc, wl.n_q), dtype=torch.int32, device="cuda")
    D.dsa_masked_mha_attn(dims, mh.dn, mh.dvh, m["q_mha"], d["kv"], k_mha, v_mha, zeros, wl.sm_scale, out, lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("name", ["tiny", "p4k_deep", "small_k", "batch2", "tiny_b3"])
def test_masked_mha_forward_bitwise_and_end_to_end(name):
    wl = CASES[name]
    mh = MhaHost(wl)
    d = SD.fill_inputs(wl)
    m = SD.fill_mha(wl)
    dims = D.Dims.of(wl)
    B, T, k = wl.batch, wl.n_q, wl.topk
    out = torch.empty((B, T, wl.heads, mh.dvh), dtype=torch.int16, device="cuda")
    lse = torch.empty((B, T, wl.heads), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, T, k), dtype=torch.int32, device="cuda")
    nws = D.dsa_masked_mha_workspace_size(dims, mh.dn, mh.dvh)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    iargs = (d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"])
    D.dsa_masked_mha_forward(dims, mh.dn, mh.dvh, *iargs, m["q_mha"], d["kv"], m["w_uk"], m["w_uv"], wl.sm_scale,
                             out, lse, idx, ws, nws)
    # chained: indexer -> top-k -> mask -> decompression -> attention
    sc = torch.empty((B, T, wl.n_kv), dtype=torch.float32, device="cuda")
    D.dsa_indexer_scores(dims, *iargs, sc, wl.n_kv)
    idx_c = torch.empty_like(idx)
    D.dsa_topk(dims, sc, wl.n_kv, idx_c)
    mask = torch.empty((B, (wl.n_kv + 31) // 32, T), dtype=torch.int32, device="cuda")
    D.dsa_selection_mask(dims, idx_c, mask)
    k_mha, v_mha = _alloc_mha(wl)
    D.dsa_mha_decompress(dims, mh.dn, mh.dvh, d["kv"], m["w_uk"], m["w_uv"], wl.q_pos0 + T, k_mha, v_mha)
    out_c, lse_c = torch.empty_like(out), torch.empty_like(lse)
    D.dsa_masked_mha_attn(dims, mh.dn, mh.dvh, m["q_mha"], d["kv"], k_mha, v_mha, mask, wl.sm_scale, out_c, lse_c)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_c) and torch.equal(out, out_c)
    assert torch.equal(lse.view(torch.int32), lse_c.view(torch.int32))
    # end to end on the GPU's (band-checked) selection
    got_idx = idx.cpu().numpy()
    rows = sorted(set(range(0, T, 9)) | {T - 1})
    for b in range(B):
        for i in rows:
            check_selection(got_idx[b, i], mh.hosts[b].scores(i), k)
    _check_rows(wl, mh, bf16_tensor_to_f64(out), lse.cpu().numpy().astype(np.float64), got_idx, rows, name + " e2e")


def test_masked_mha_simulates_sparse_mqa_attention():
    # The two MLA forms agree on the GPU as well: masked MHA mode on the
    # selection equals W_UV[h] applied to the sparse MQA-mode attention of
    # the absorbed query [W_UK[h]^T q_nope | q_rope] (rounded to bf16).
    wl = CASES["p4k_deep"]
    mh = MhaHost(wl)
    d = SD.fill_inputs(wl)
    m = SD.fill_mha(wl)
    dims = D.Dims.of(wl)
    sel = _oracle_selection(wl, mh)
    idx = torch.from_numpy(sel).cuda()
    mask = torch.empty((1, (wl.n_kv + 31) // 32, wl.n_q), dtype=torch.int32, device="cuda")
    D.dsa_selection_mask(dims, idx, mask)
    k_mha, v_mha = _alloc_mha(wl)
    D.dsa_mha_decompress(dims, mh.dn, mh.dvh, d["kv"], m["w_uk"], m["w_uv"], wl.q_pos0 + wl.n_q, k_mha, v_mha)
    out = torch.empty((1, wl.n_q, wl.heads, mh.dvh), dtype=torch.int16, device="cuda")
    D.dsa_masked_mha_attn(dims, mh.dn, mh.dvh, m["q_mha"], d["kv"], k_mha, v_mha, mask, wl.sm_scale, out)
    # absorbed queries (host, fp64 -> bf16) through the sparse MQA kernel
    qm = np.stack([mh.q_mha(0, i) for i in range(wl.n_q)])                          # [T, H, dn + dr]
    q_abs = np.concatenate([np.einsum("hdc,thd->thc", mh.w_uk, qm[:, :, :mh.dn]), qm[:, :, mh.dn:]], axis=2)
    from synth import gen
    q_abs_dev = torch.from_numpy(gen.f32_to_bf16_bits(q_abs.astype(np.float32)).view(np.int16)[None]).cuda()
    o_lat = torch.empty((1, wl.n_q, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    nws = D.dsa_attn_workspace_size(dims)
    aws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    D.dsa_sparse_mla_attn(dims, q_abs_dev, d["kv"], idx, wl.sm_scale, o_lat, None, aws, nws)
    torch.cuda.synchronize()
    proj = np.einsum("hdc,thc->thd", mh.w_uv, bf16_tensor_to_f64(o_lat)[0])
    got = bf16_tensor_to_f64(out)[0]
    worst = 0.0
    for i in range(wl.n_q):
        err = attn_errors(got[i], proj[i])
        assert np.all(err <= 2 * ATTN_MAX_REL), (i, float(err.max()))
        worst = max(worst, float(err.max()))
    _say("MHA vs absorbed MQA on the GPU: max rel diff", worst)


def test_masked_mha_full_size_sampled():
    # 4096-token prefill at its real shape (128 heads, k = 2048), through the
    # fused call as the benchmark times it; sampled rows against the oracle.
    wl = W.WORKLOADS["p4k"]
    mh = MhaHost(wl)
    d = SD.fill_inputs(wl)
    m = SD.fill_mha(wl)
    dims = D.Dims.of(wl)
    T, k = wl.n_q, wl.topk
    out = torch.empty((1, T, wl.heads, mh.dvh), dtype=torch.int16, device="cuda")
    lse = torch.empty((1, T, wl.heads), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, T, k), dtype=torch.int32, device="cuda")
    nws = D.dsa_masked_mha_workspace_size(dims, mh.dn, mh.dvh)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    D.dsa_masked_mha_forward(dims, mh.dn, mh.dvh, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"],
                             m["q_mha"], d["kv"], m["w_uk"], m["w_uv"], wl.sm_scale, out, lse, idx, ws, nws)
    torch.cuda.synchronize()
    got_idx = idx.cpu().numpy()
    rows = [0, 1, 31, 32, 127, 128, 1000, 2047, 2048, 2049, 3001, 4095]
    for i in rows:
        check_selection(got_idx[0, i], mh.hosts[0].scores(i), k)
    mh.kvh(0, wl.n_kv)
    _check_rows(wl, mh, bf16_tensor_to_f64(out), lse.cpu().numpy().astype(np.float64), got_idx, rows, "p4k full")
