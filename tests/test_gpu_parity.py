"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Small workloads are compared everywhere; the full-size
workloads run in the configuration the benchmark times and are compared on
sampled rows that the oracle computes one by one."""
import zlib

import numpy as np
import pytest
import torch

import sparse_attention_long_amd as dsa
from oracle import dsa_oracle as O
from synth import workloads as W
from synth import device as SD

from dsa_parity import (ATTN_MAX_REL, LSE_ABS, SCORE_REL_RMS, HostSide, attn_errors, bf16_tensor_to_f64,
                        check_selection, score_rel_rms, to_dev)

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


def host_dev_inputs(wl):
    h = W.host_inputs(wl)
    return h, {k: to_dev(v) for k, v in h.items()}


def run_indexer(wl, d, ld=None, sentinel=float("nan")):
    ld = ld or wl.n_kv
    sc = torch.full((wl.batch, wl.n_q, ld), sentinel, dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores(dsa.Dims.of(wl), d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], sc, ld)
    torch.cuda.synchronize()
    return sc


def sample_rows(T, extra=()):
    rows = {0, 1, 15, 16, 31, 32, 33, 63, 64, T // 2, T - 33, T - 32, T - 17, T - 2, T - 1, *extra}
    return sorted(r for r in rows if 0 <= r < T)


# ----------------------------------------------------------------- generator
def test_device_generator_matches_host():
    tiny = W.WORKLOADS["tiny"]
    h = W.host_inputs(tiny)
    d = SD.fill_inputs(tiny)
    torch.cuda.synchronize()
    for k, v in h.items():
        got = d[k].cpu().numpy()
        assert np.array_equal(got.view(v.dtype) if v.dtype == np.uint16 else got, v), k
    wl = W.WORKLOADS["p4k"]
    d = SD.fill_inputs(wl)
    torch.cuda.synchronize()
    rows = [0, 1, 1234, 4095]
    c, s = W.q_idx_fp8(wl, 0, rows)
    assert np.array_equal(d["q_idx"][0, rows].cpu().numpy(), c)
    assert np.array_equal(d["q_scale"][0, rows].cpu().numpy(), s)
    assert np.array_equal(d["q"][0, rows].cpu().numpy().view(np.uint16), W.q_bf16(wl, 0, rows))
    assert np.array_equal(d["w_idx"][0].cpu().numpy().view(np.uint16), W.w_idx_bf16(wl, 0, range(4096)))
    c, s = W.k_idx_fp8(wl, 0, 0, 4096)
    assert np.array_equal(d["k_idx"][0].cpu().numpy(), c) and np.array_equal(d["k_scale"][0].cpu().numpy(), s)
    assert np.array_equal(d["kv"][0, rows].cpu().numpy().view(np.uint16), W.kv_bf16_rows(wl, 0, rows))


# ----------------------------------------------------------------- indexer
def test_indexer_tiny_all_rows():
    wl = W.WORKLOADS["tiny"]
    h, d = host_dev_inputs(wl)
    sc = run_indexer(wl, d).cpu().numpy()
    hs = HostSide(wl)
    pairs = []
    for i in range(wl.n_q):
        n = min(i + 1, wl.n_kv)
        ref = hs.scores(i)
        pairs.append((sc[0, i, :n], ref))
        assert np.all(np.isnan(sc[0, i, n:])), f"row {i}: wrote beyond the causal window"
    err = score_rel_rms(pairs)
    _say("tiny indexer rel RMS", err)
    assert err <= SCORE_REL_RMS


INDEXER_CASES = {
    "p4k": W.WORKLOADS["p4k"],
    "ragged_3001": W.custom("p4k", n_q=3001, n_kv=3001),
    "chunk_pos0": W.custom("p4k", n_q=700, n_kv=3095, q_pos0=2395),
    "rows5": W.custom("p4k", n_q=5, n_kv=1037, q_pos0=1032),
    "decode_b3": W.custom("dec64", batch=3, n_kv=5003, q_pos0=5002),
    "decode_t3": W.custom("dec64", batch=2, n_q=3, n_kv=4099, q_pos0=4096),
    # two forward chunks at 65536 keys (1024 rows, then a ragged 512)
    "two_chunks": W.custom("p4k", n_q=1536, n_kv=65536, q_pos0=64000),
    # few long decode rows: the fused forward spreads each row's top-k over
    # several workgroups (odd length: ragged vector split and scalar tail)
    "decode_long_b4": W.custom("dec64", batch=4, n_kv=20011, q_pos0=20010),
    "decode_long_t3": W.custom("dec64", batch=2, n_q=3, n_kv=33000, q_pos0=32997),
}


@pytest.mark.parametrize("name", list(INDEXER_CASES))
def test_indexer_production_dims(name):
    wl = INDEXER_CASES[name]
    d = SD.fill_inputs(wl)
    ld = wl.n_kv + 7
    sc = run_indexer(wl, d, ld=ld)
    pairs = []
    for b in sorted({0, wl.batch - 1}):
        hs = HostSide(wl, b)
        for i in sample_rows(wl.n_q):
            n = min(wl.q_pos0 + i + 1, wl.n_kv)
            row = sc[b, i].cpu().numpy()
            assert not np.any(np.isnan(row[:n])), (b, i)
            assert np.all(np.isnan(row[n:])), (b, i)
            pairs.append((row[:n], hs.scores(i)))
    err = score_rel_rms(pairs)
    _say(name, "indexer rel RMS", err)
    assert err <= SCORE_REL_RMS


# ----------------------------------------------------------------- top-k
def run_topk(scores_np, k, pos0=None):
    B, T, S = scores_np.shape
    pos0 = S - T if pos0 is None else pos0
    dims = dsa.Dims(batch=B, n_q=T, n_kv=S, q_pos0=pos0, idx_heads=64, idx_dim=128, heads=128, dim_qk=576,
                    dim_v=512, topk=k)
    idx = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(dims, to_dev(scores_np.astype(np.float32)), S, idx)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def assert_topk_exact(scores_np, k, pos0=None):
    B, T, S = scores_np.shape
    pos0 = S - T if pos0 is None else pos0
    got = run_topk(scores_np, k, pos0)
    for b in range(B):
        for i in range(T):
            n = min(pos0 + i + 1, S)
            want = O.topk_row(scores_np[b, i, :n], k)
            assert np.array_equal(got[b, i], want), (b, i, n)


def test_topk_rows_shorter_than_the_sample():
    # rows with k < n < 64 take no sampled cutoff (its 64-score blocks do not
    # fit) and collect every score; the scores buffer is its own allocation
    rs = np.random.RandomState(11)
    for k, S, pos0, T in ((8, 40, 10, 30), (1, 63, 0, 63), (32, 70, 40, 30)):
        sc = rs.randn(1, T, S).astype(np.float32)
        sc[0, :, ::5] = 0.25   # ties
        assert_topk_exact(sc, k, pos0)


def test_topk_ws_equals_topk():
    # few long rows: with a workspace the collection is split over several
    # workgroups per row; the selection is the same bit for bit
    rs = np.random.RandomState(12)
    for B, T, S, k in ((4, 1, 20011, 2048), (2, 3, 33000, 2048), (64, 1, 131072, 2048)):
        x = rs.randn(B, T, S).astype(np.float32)
        x[:, :, 100:3000:3] = 1.5   # a block of ties near the cutoff
        dims = dsa.Dims(batch=B, n_q=T, n_kv=S, q_pos0=S - T, idx_heads=64, idx_dim=128, heads=128, dim_qk=576,
                        dim_v=512, topk=k)
        nws = dsa.dsa.dsa_topk_workspace_size(dims)
        assert nws > 0
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        xs = to_dev(x)
        a = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
        c = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
        dsa.dsa_topk(dims, xs, S, a)
        dsa.dsa.dsa_topk_ws(dims, xs, S, c, ws, nws)
        torch.cuda.synchronize()
        assert torch.equal(a, c), (B, T, S)
        want = O.topk_row(x[B - 1, T - 1], k)
        assert np.array_equal(c[B - 1, T - 1].cpu().numpy(), want)


def test_topk_ws_candidates_in_few_parts():
    # Rows whose candidates all sit in one or two of the split collection's
    # parts: the merge assembles each thread's slice of the candidate list
    # from the parts, skipping the empty ones.  Increasing scores put every
    # candidate in the last part, decreasing in the first, a V shape in the
    # two end parts with empty parts between, a bump in the middle parts.
    # The sampled cutoff keeps about 2k candidates: with k = 512 they fit one
    # part's list (8 parts per row here); with k = 2048 a single part's list
    # can overflow, and the merge falls back to its own pass over the row.
    rs = np.random.RandomState(14)
    for B, S, k in ((8, 65536, 512), (64, 131072, 2048)):
        T = 1
        j = np.arange(S, dtype=np.float64)
        shapes = [j, S - j, np.abs(j - S / 2), -np.abs(j - S / 2)]
        x = np.stack([shapes[b % 4] + 0.25 * rs.rand(S) for b in range(B)]).astype(np.float32)[:, None, :]
        dims = dsa.Dims(batch=B, n_q=T, n_kv=S, q_pos0=S - T, idx_heads=64, idx_dim=128, heads=128, dim_qk=576,
                        dim_v=512, topk=k)
        nws = dsa.dsa.dsa_topk_workspace_size(dims)
        assert nws > 0
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        xs = to_dev(x)
        a = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
        c = torch.full((B, T, k), -7, dtype=torch.int32, device="cuda")
        dsa.dsa_topk(dims, xs, S, a)
        dsa.dsa.dsa_topk_ws(dims, xs, S, c, ws, nws)
        torch.cuda.synchronize()
        assert torch.equal(a, c), (B, S)
        got = c.cpu().numpy()
        for b in range(4):
            assert np.array_equal(got[b, 0], O.topk_row(x[b, 0], k)), (B, S, b)
        _say("split top-k, candidates in few parts", B, "rows of", S, "keys: equal to dsa_topk and the oracle")


def test_validate_counts_planted_values():
    """dsa_validate counts exactly the bad values planted on the host."""
    D = dsa.dsa
    B, T, S, k, HI = 3, 4, 300, 16, 64
    rs = np.random.RandomState(13)
    dims = dsa.Dims(batch=B, n_q=T, n_kv=S, q_pos0=S - T, idx_heads=HI, idx_dim=128, heads=128, dim_qk=576,
                    dim_v=512, topk=k)
    qs = rs.rand(B, T).astype(np.float32) + 0.5
    w = np.full((B, T, HI), 0x3F80, np.uint16)          # bf16 1.0
    ks = rs.rand(B, S).astype(np.float32) + 0.5
    idx = np.stack([np.stack([np.sort(rs.choice(S - T + i + 1, k, replace=False)) for i in range(T)])
                    for _ in range(B)]).astype(np.int32)
    counts = torch.full((8,), -1, dtype=torch.int32, device="cuda")

    def run(layout=None, **kw):
        a = dict(q_scale=qs, w=w, k_scale=ks, idx=idx)
        a.update(kw)
        D.dsa_validate(dims, layout, to_dev(a["q_scale"]), to_dev(a["w"]), to_dev(a["k_scale"]), to_dev(a["idx"]),
                       counts)
        torch.cuda.synchronize()
        return counts.cpu().numpy().tolist()

    assert run() == [0] * 8
    q2 = qs.copy(); q2[0, 1] = np.nan; q2[2, 3] = 0.0; q2[1, 0] = -1.0; q2[1, 1] = np.inf
    w2 = w.copy(); w2[1, 2, 5] = 0x7FC0; w2[0, 0, 63] = 0xFF80                   # NaN, -inf
    k2 = ks.copy(); k2[0, 0] = np.nan; k2[2, S - 1] = -2.0; k2[1, 77] = 0.0
    i2 = idx.copy()
    i2[0, 0, 3] = S - T + 1        # past row 0's window (n_p = S - T + 1): out of range, and order broken
    i2[1, 2, 0] = -5               # out of range
    i2[2, 1, 5] = i2[2, 1, 4]      # duplicate: not canonical
    i2[2, 3, 10:] = -1             # canonical padding
    i2[0, 2, 7] = -1               # a hole: valid entries after -1
    got = run(q_scale=q2, w=w2, k_scale=k2, idx=i2)
    # rows (0, 0), (2, 1) and (0, 2) are not canonical; -5 counts as out of range only
    assert got == [4, 2, 3, 2, 3, 0, 0, 0], got
    # variable-length layout: lengths and page entries
    lens = np.array([S, S - 50, T - 1], np.int32)        # the last one is below n_q
    table = np.array([[0, 1, 2, 3, 4], [5, 6, 99, 7, 8], [9, -1, 10, 11, 12]], np.int32)   # 64-token pages
    lens_d, table_d = to_dev(lens), to_dev(table)   # kept alive: the layout holds raw pointers
    lay = D.PagedKV.of(lens_d, table_d, 64, 5, 16)
    pool_ks = (rs.rand(16 * 64).astype(np.float32) + 0.5)
    idx_v = np.full((B, T, k), -1, np.int32)
    got = run(layout=lay, k_scale=pool_ks, idx=idx_v)
    # seq 1 uses ceil(250/64) = 4 pages (entry 99 is bad); seq 2 is clamped to
    # n_q = 4 tokens: one page, entry 9, fine
    assert got == [0, 0, 0, 0, 0, 1, 1, 0], got


def test_topk_exact_on_oracle_scores_tiny():
    wl = W.WORKLOADS["tiny"]
    hs = HostSide(wl)
    sc = np.full((1, wl.n_q, wl.n_kv), np.nan, np.float32)
    for i in range(wl.n_q):
        sc[0, i, :i + 1] = hs.scores(i)
    assert_topk_exact(sc, wl.topk, 0)


def test_topk_exact_on_oracle_scores_production():
    wl = W.custom("p4k", n_q=96, n_kv=6000, q_pos0=5904)
    hs = HostSide(wl)
    sc = np.full((1, wl.n_q, wl.n_kv), np.nan, np.float32)
    for i in range(wl.n_q):
        sc[0, i, :wl.q_pos0 + i + 1] = hs.scores(i)
    assert_topk_exact(sc, 2048)


@pytest.mark.parametrize("case", ["ties_small_ints", "nan_and_zeros", "all_equal", "wide_bin", "k_plus_one",
                                  "negative", "k1", "long_rows"])
def test_topk_exact_adversarial(case):
    rs = np.random.RandomState(zlib.crc32(case.encode()))
    if case == "ties_small_ints":
        sc, k = np.round(rs.randn(2, 40, 5000) * 2).astype(np.float32), 300
    elif case == "nan_and_zeros":
        sc = rs.randn(1, 20, 3000).astype(np.float32)
        sc[rs.rand(*sc.shape) < 0.3] = np.nan
        sc[rs.rand(*sc.shape) < 0.3] = 0.0
        sc[rs.rand(*sc.shape) < 0.3] = -0.0
        k = 2048
    elif case == "all_equal":
        sc, k = np.full((1, 8, 9000), 1.5, np.float32), 2048
    elif case == "wide_bin":   # one top-11-bit bin holds > 4096 keys: multi-pass path
        sc = (1.0 + rs.rand(1, 6, 30000) * 0.2).astype(np.float32)
        sc[0, :, ::7] = 1.1          # exact ties inside the wide bin
        k = 2048
    elif case == "k_plus_one":
        sc, k = rs.randn(1, 3, 2049).astype(np.float32), 2048
    elif case == "negative":
        sc, k = (-np.abs(rs.randn(1, 10, 4000)) * 1e-30).astype(np.float32), 1000
    elif case == "k1":
        sc, k = rs.randn(3, 5, 777).astype(np.float32), 1
    else:
        sc, k = rs.randn(1, 4, 131072).astype(np.float32), 2048
    assert_topk_exact(sc, k)


# ----------------------------------------------------------------- attention
def run_attn(wl, q_dev, kv_dev, idx_np, rows):
    dims = dsa.Dims.of(wl, n_q=rows, q_pos0=0)
    B = wl.batch
    out = torch.zeros((B, rows, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    lse = torch.zeros((B, rows, wl.heads), dtype=torch.float32, device="cuda")
    nws = dsa.dsa_attn_workspace_size(dims)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_sparse_mla_attn(dims, q_dev, kv_dev, to_dev(idx_np.astype(np.int32)), wl.sm_scale, out, lse, ws, nws)
    torch.cuda.synchronize()
    return bf16_tensor_to_f64(out), lse.cpu().numpy(), nws


def _attn_case(wl, rows, sel_of_row, q_mul=1.0):
    """Attention only: q rows chosen by `rows` (positions 0.. of a [1, len(rows)] call)."""
    B = wl.batch
    hs = [HostSide(wl, b) for b in range(B)]
    q = np.stack([np.stack([W.q_bf16(wl, b, [i])[0] for i in rows]) for b in range(B)])
    if q_mul != 1.0:
        from synth import gen
        q = np.stack([gen.f32_to_bf16_bits(O.bf16_decode(q[b]).astype(np.float32) * np.float32(q_mul)) for b in range(B)])
    idx = np.stack([np.stack([sel_of_row(b, i) for i in rows]) for b in range(B)])
    kv = np.stack([W.kv_bf16_rows(wl, b, np.arange(wl.n_kv)) for b in range(B)])
    o, lse, nws = run_attn(wl, to_dev(q), to_dev(kv), idx, len(rows))
    worst, worst_lse = 0.0, 0.0
    for b in range(B):
        for n, i in enumerate(rows):
            qv = O.bf16_decode(q[b, n])
            kvf = O.bf16_decode(kv[b])
            ref_o, ref_lse = O.sparse_mla_row(qv, kvf, idx[b, n], wl.sm_scale, wl.dim_v)
            if not np.any(idx[b, n] >= 0):
                assert np.all(o[b, n] == 0) and np.all(np.isneginf(lse[b, n]))
                continue
            worst = max(worst, attn_errors(o[b, n], ref_o).max())
            worst_lse = max(worst_lse, np.abs(lse[b, n] - ref_lse).max())
    return worst, worst_lse, nws


def test_attention_tiny_oracle_selection():
    wl = W.WORKLOADS["tiny"]
    hs = HostSide(wl)
    worst, wl_lse, _ = _attn_case(wl, list(range(wl.n_q)), lambda b, i: O.topk_row(hs.scores(i), wl.topk))
    _say("tiny attention max rel err", worst, "lse abs err", wl_lse)
    assert worst <= ATTN_MAX_REL and wl_lse <= LSE_ABS


def test_attention_production_dims_rows():
    wl = W.custom("p4k", n_kv=4096)
    hs = HostSide(wl)
    rows = [0, 1, 31, 32, 100, 2046, 2047, 2048, 3000, 4095]
    worst, wlse, nws = _attn_case(wl, rows, lambda b, i: O.topk_row(hs.scores(i), wl.topk))
    _say("p4k rows attention max rel err", worst, "lse", wlse, "ws", nws)
    assert worst <= ATTN_MAX_REL and wlse <= LSE_ABS


def test_attention_split_path_and_padding():
    # few rows -> the selected set is split across workgroups and merged
    wl = W.custom("dec64", batch=4, n_kv=9000, q_pos0=8999)
    rs = np.random.RandomState(3)

    def sel(b, i):
        m = [2048, 1500, 37, 0][b]
        out = np.full(2048, -1, np.int32)
        out[:m] = np.sort(rs.choice(9000, size=m, replace=False))
        return out

    worst, wlse, nws = _attn_case(wl, [0], sel)
    _say("split attention max rel err", worst, "lse", wlse, "ws", nws)
    assert nws > 0
    assert worst <= ATTN_MAX_REL and wlse <= LSE_ABS


def test_attention_large_logits_recompute_path():
    # logits far above the first chunk's maximum force the second pass
    wl = W.custom("p4k", n_kv=4096)
    rs = np.random.RandomState(4)
    worst, wlse, _ = _attn_case(wl, [5, 6, 7], lambda b, i: np.sort(rs.choice(4096, 2048, replace=False)).astype(np.int32),
                                q_mul=40.0)
    _say("large-logit attention max rel err", worst, "lse", wlse)
    assert worst <= ATTN_MAX_REL and wlse <= LSE_ABS * 40


def test_attention_large_logits_recompute_path_unsplit():
    # 256 rows: one workgroup per row (no split), each row forced into the
    # second pass by logits far above its first chunk's maximum
    wl = W.custom("p4k", n_kv=4096)
    rs = np.random.RandomState(5)
    rows = list(range(256))
    dims = dsa.Dims.of(wl, n_q=len(rows), q_pos0=0)
    assert dsa.dsa_attn_workspace_size(dims) == 0
    worst, wlse, _ = _attn_case(wl, rows, lambda b, i: np.sort(rs.choice(4096, 2048, replace=False)).astype(np.int32),
                                q_mul=40.0)
    _say("large-logit unsplit attention max rel err", worst, "lse", wlse)
    assert worst <= ATTN_MAX_REL and wlse <= LSE_ABS * 40


@pytest.mark.parametrize("heads,rows", [(72, 3), (72, 256), (1, 2), (100, 300)])
def test_attention_head_counts_not_multiple_of_32(heads, rows):
    # A wave owns 32 heads, and the output leaves through a per-wave staging
    # buffer in whole head rows: heads past H must be neither computed into
    # the output nor stored.  rows < 256 takes the split path (partials and
    # the combine), rows >= 256 one workgroup per row.  The output sits at
    # the start of a larger buffer whose tail must stay untouched.
    wl = W.custom("p4k", n_kv=4096, heads=heads)
    rs = np.random.RandomState(11 + heads + rows)
    q = np.stack([W.q_bf16(wl, 0, [i])[0] for i in range(rows)])[None]
    idx = np.stack([np.sort(rs.choice(4096, 2048, replace=False)).astype(np.int32) for _ in range(rows)])[None]
    kv = W.kv_bf16_rows(wl, 0, np.arange(wl.n_kv))[None]
    dims = dsa.Dims.of(wl, n_q=rows, q_pos0=0)
    n_out = rows * heads * wl.dim_v
    guard = 64 * wl.dim_v
    buf = torch.full((n_out + guard,), 0x7F7F, dtype=torch.int16, device="cuda")
    out = buf[:n_out].view(1, rows, heads, wl.dim_v)
    lse = torch.zeros((1, rows, heads), dtype=torch.float32, device="cuda")
    nws = dsa.dsa_attn_workspace_size(dims)
    assert (nws > 0) == (rows < 256)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_sparse_mla_attn(dims, to_dev(q), to_dev(kv), to_dev(idx), wl.sm_scale, out, lse, ws, nws)
    torch.cuda.synchronize()
    assert bool(torch.all(buf[n_out:] == 0x7F7F)), "store past the last head"
    o = bf16_tensor_to_f64(out)
    l = lse.cpu().numpy()
    kvf = O.bf16_decode(kv[0])
    check = sorted(set(range(rows)) if rows <= 8 else {0, 1, 31, 32, 100, rows // 2, rows - 2, rows - 1})
    worst, worst_lse = 0.0, 0.0
    for n in check:
        ref_o, ref_lse = O.sparse_mla_row(O.bf16_decode(q[0, n]), kvf, idx[0, n], wl.sm_scale, wl.dim_v)
        worst = max(worst, attn_errors(o[0, n], ref_o).max())
        worst_lse = max(worst_lse, np.abs(l[0, n] - ref_lse).max())
    _say(f"H={heads} rows={rows} ws={nws}: attention max rel err", worst, "lse", worst_lse, "rows checked", len(check))
    assert worst <= ATTN_MAX_REL and worst_lse <= LSE_ABS


# ----------------------------------------------------------------- fused forward
def run_forward(wl, d, with_idx=True):
    dims = dsa.Dims.of(wl)
    out = torch.empty((wl.batch, wl.n_q, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.batch, wl.n_q, wl.heads), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.batch, wl.n_q, wl.topk), dtype=torch.int32, device="cuda") if with_idx else None
    nws = dsa.dsa_forward_workspace_size(dims)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    dsa.dsa_forward(dims, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], d["q"], d["kv"],
                    wl.sm_scale, out, lse, idx, ws, nws)
    torch.cuda.synchronize()
    return out, lse, idx


@pytest.mark.parametrize("name", ["tiny", "p4k", "decode_b3", "chunk_pos0", "two_chunks", "decode_long_b4",
                                  "decode_long_t3"])
def test_forward_bitwise_equals_chained_calls(name):
    wl = W.WORKLOADS.get(name) or INDEXER_CASES[name]
    d = SD.fill_inputs(wl)
    out, lse, idx = run_forward(wl, d)
    out2, lse2, _ = run_forward(wl, d, with_idx=False)
    dims = dsa.Dims.of(wl)
    sc = run_indexer(wl, d)
    idx_c = torch.empty_like(idx)
    dsa.dsa_topk(dims, sc, wl.n_kv, idx_c)
    out_c = torch.empty_like(out)
    lse_c = torch.empty_like(lse)
    nws = dsa.dsa_attn_workspace_size(dims)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_sparse_mla_attn(dims, d["q"], d["kv"], idx_c, wl.sm_scale, out_c, lse_c, ws, nws)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_c)
    assert torch.equal(out, out_c) and torch.equal(out, out2)
    assert torch.equal(lse.view(torch.int32), lse_c.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


def chained_forward(wl, d):
    """dsa_indexer_scores, dsa_topk and dsa_sparse_mla_attn one after the other."""
    dims = dsa.Dims.of(wl)
    sc = run_indexer(wl, d)
    idx_c = torch.empty((wl.batch, wl.n_q, wl.topk), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(dims, sc, wl.n_kv, idx_c)
    del sc
    out_c = torch.empty((wl.batch, wl.n_q, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    lse_c = torch.empty((wl.batch, wl.n_q, wl.heads), dtype=torch.float32, device="cuda")
    nws = dsa.dsa_attn_workspace_size(dims)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_sparse_mla_attn(dims, d["q"], d["kv"], idx_c, wl.sm_scale, out_c, lse_c, ws, nws)
    torch.cuda.synchronize()
    return out_c, lse_c, idx_c


def assert_forward_equals_chained(wl, d):
    out, lse, idx = run_forward(wl, d)
    out_c, lse_c, idx_c = chained_forward(wl, d)
    assert torch.equal(idx, idx_c)
    assert torch.equal(out, out_c)
    assert torch.equal(lse.view(torch.int32), lse_c.view(torch.int32))
    return idx


def test_forward_all_scores_equal():
    """Every key identical: all of a row's 64,000+ scores are equal, the
    sampled cutoff collects every key (far more than the candidate list
    holds) and each row takes the two-pass fallback.  Still the chained
    result, and the ties go to the lowest indices (analysis page, Sec. 5.2:
    equal scores at the cutoff are legitimate)."""
    wl = INDEXER_CASES["two_chunks"]
    d = SD.fill_inputs(wl)
    d["k_idx"].fill_(0x38)     # e4m3 1.0
    d["k_scale"].fill_(1.0)
    idx = assert_forward_equals_chained(wl, d)
    want = torch.arange(wl.topk, dtype=torch.int32, device="cuda").expand(wl.batch, wl.n_q, wl.topk)
    assert torch.equal(idx, want)


def test_forward_long_prefill_from_position_zero():
    """A 20480-token prefill from position 0 in chunks of 3264 rows: short
    and long rows, a ragged last chunk; the whole result is the chained
    one."""
    wl = W.custom("p4k", n_q=20480, n_kv=20480, q_pos0=0)
    plan = dsa.dsa.dsa_forward_plan_of(dsa.Dims.of(wl))
    assert plan.chunk_rows == 3264 and wl.n_q % plan.chunk_rows != 0
    d = SD.fill_inputs(wl)
    assert_forward_equals_chained(wl, d)


def test_forward_ordered_on_caller_stream():
    """Rows spanning several chunks all run on the caller's stream.  Work
    enqueued on that stream just before the call (the query copy) must be
    seen by every chunk, and work enqueued just after it (the snapshots) must
    see every chunk's results."""
    wl = INDEXER_CASES["two_chunks"]   # chunks of 1024 and 512 rows at 65,536 keys
    d = SD.fill_inputs(wl)
    ref_out, ref_lse, ref_idx = run_forward(wl, d)
    dims = dsa.Dims.of(wl)
    nws = dsa.dsa_forward_workspace_size(dims)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    snaps = []
    with torch.cuda.stream(side):
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        q_in = torch.zeros_like(d["q"])
        out, lse, idx = torch.empty_like(ref_out), torch.empty_like(ref_lse), torch.empty_like(ref_idx)
        for rep in range(3):
            q_in.zero_()
            out.fill_(0)
            idx.fill_(-1)
            q_in.copy_(d["q"])
            dsa.dsa_forward(dims, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], q_in, d["kv"],
                            wl.sm_scale, out, lse, idx, ws, nws)
            snaps.append((out.clone(), lse.clone(), idx.clone()))
    torch.cuda.synchronize()
    for o, l, i in snaps:
        assert torch.equal(i, ref_idx)
        assert torch.equal(o, ref_out)
        assert torch.equal(l.view(torch.int32), ref_lse.view(torch.int32))


def test_forward_graph_replays_match_eager():
    """A multi-chunk dsa_forward captured into a graph: every replay, with
    eager work and synchronisations between replays, equals the eager call."""
    wl = INDEXER_CASES["two_chunks"]
    d = SD.fill_inputs(wl)
    ref_out, ref_lse, ref_idx = run_forward(wl, d)   # eager
    dims = dsa.Dims.of(wl)
    nws = dsa.dsa_forward_workspace_size(dims)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    out, lse, idx = torch.empty_like(ref_out), torch.empty_like(ref_lse), torch.empty_like(ref_idx)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dsa.dsa_forward(dims, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], d["q"], d["kv"],
                        wl.sm_scale, out, lse, idx, ws, nws)
    for rep in range(4):
        out.fill_(0)
        lse.fill_(0)
        idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say("graph replay", rep)
        assert torch.equal(idx, ref_idx)
        assert torch.equal(out, ref_out)
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        o2, _, _ = run_forward(wl, d, with_idx=False)   # eager work between replays
        assert torch.equal(o2, ref_out)


def test_forward_from_two_host_threads():
    """Two host threads run multi-chunk forwards at once, each on its own
    stream and workspace; every result equals the one-thread result."""
    import threading
    wl = INDEXER_CASES["two_chunks"]
    d = SD.fill_inputs(wl)
    ref_out, ref_lse, ref_idx = run_forward(wl, d)
    dims = dsa.Dims.of(wl)
    nws = dsa.dsa_forward_workspace_size(dims)
    bufs = [(torch.empty(nws, dtype=torch.uint8, device="cuda"), torch.empty_like(ref_out),
             torch.empty_like(ref_lse), torch.empty_like(ref_idx), torch.cuda.Stream()) for _ in range(2)]
    torch.cuda.synchronize()
    errors, results = [], [[] for _ in bufs]

    def worker(t):
        try:
            ws, out, lse, idx, st = bufs[t]
            with torch.cuda.stream(st):
                for _ in range(3):
                    dsa.dsa_forward(dims, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], d["q"],
                                    d["kv"], wl.sm_scale, out, lse, idx, ws, nws)
                    results[t].append((out.clone(), lse.clone(), idx.clone()))
            st.synchronize()
        except Exception as e:   # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    torch.cuda.synchronize()
    assert not errors, errors
    assert all(len(r) == 3 for r in results)
    for r in results:
        for o, l, i in r:
            assert torch.equal(i, ref_idx)
            assert torch.equal(o, ref_out)
            assert torch.equal(l.view(torch.int32), ref_lse.view(torch.int32))


def test_forward_split_topk_fallback_on_equal_scores():
    # All-zero index keys make every score 0: every key is a candidate, each
    # of the fused forward's top-k parts overflows its candidate list, and
    # the merge takes the two-pass fallback.  Ties go to the lower index, so
    # every row selects 0 .. k-1, as the chained calls do.
    wl = W.custom("dec64", batch=2, n_kv=20000, q_pos0=19999)
    d = SD.fill_inputs(wl)
    d["k_idx"].zero_()
    out, lse, idx = run_forward(wl, d)
    want = torch.arange(wl.topk, dtype=torch.int32, device="cuda").expand(wl.batch, wl.n_q, wl.topk)
    assert torch.equal(idx, want)
    dims = dsa.Dims.of(wl)
    sc = run_indexer(wl, d)
    assert torch.all(sc == 0)
    idx_c = torch.empty_like(idx)
    dsa.dsa_topk(dims, sc, wl.n_kv, idx_c)
    out_c, lse_c = torch.empty_like(out), torch.empty_like(lse)
    nws = dsa.dsa_attn_workspace_size(dims)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_sparse_mla_attn(dims, d["q"], d["kv"], idx_c, wl.sm_scale, out_c, lse_c, ws, nws)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx_c) and torch.equal(out, out_c)
    assert torch.equal(lse.view(torch.int32), lse_c.view(torch.int32))


def check_forward_rows(wl, out, lse, idx, rows_by_seq):
    """Every listed row: the GPU selection against the oracle scores (band
    rule), then the oracle attention over that same GPU selection against the
    GPU's output.  Every row is compared; returns the worst errors, the mean
    recall, the ambiguous positions and the number of rows compared."""
    worst, worst_lse, recall, amb, compared = 0.0, 0.0, [], 0, 0
    for b, rows in rows_by_seq.items():
        hs = HostSide(wl, b)
        for i in rows:
            gsel = idx[b, i].cpu().numpy()
            r, a = check_selection(gsel, hs.scores(i), wl.topk)
            recall.append(r); amb += a
            ref_o, ref_lse = hs.attention(i, gsel)
            o = bf16_tensor_to_f64(out[b, i])
            worst = max(worst, attn_errors(o, ref_o).max())
            worst_lse = max(worst_lse, np.abs(lse[b, i].cpu().numpy() - ref_lse).max())
            compared += 1
    return worst, worst_lse, float(np.mean(recall)), amb, compared


def test_forward_tiny_end_to_end():
    wl = W.WORKLOADS["tiny"]
    out, lse, idx = run_forward(wl, SD.fill_inputs(wl))
    worst, wlse, rec, amb, n = check_forward_rows(wl, out, lse, idx, {0: range(wl.n_q)})
    _say("tiny forward: attn err", worst, "lse", wlse, "recall", rec, "ambiguous", amb, "rows compared", n)
    assert n == wl.n_q
    assert worst <= ATTN_MAX_REL and wlse <= LSE_ABS


# ----------------------------------------------------------------- full size (sampled rows)
FULL = ["p4k", "p32k", "p128k", "dec64"]


def stratified_rows(T, R):
    """R stratified rows floor((r + 1/2) T / R) plus the last row."""
    return sorted({int((r + 0.5) * T / R) for r in range(R)} | {T - 1})


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name", FULL)
def test_forward_full_size_sampled(name):
    """The full workload through dsa_forward in the configuration the
    benchmark times, checked on rows the oracle computes one by one (in a
    pool of worker processes): all 64 decode rows; 1024 stratified rows plus
    the last at 128K; 512 plus the last at 4K and 32K (rows below k = 2048
    are the dense-equivalence cases)."""
    import oracle_pool
    wl = W.WORKLOADS[name]
    d = SD.fill_inputs(wl)
    out, lse, idx = run_forward(wl, d)
    del d
    if wl.n_q == 1:
        rows = {b: [0] for b in range(wl.batch)}
    else:
        rows = {0: stratified_rows(wl.n_q, 1024 if wl.n_q >= 131072 else 512)}
    _say(name, "forward done; oracle rows", sum(len(r) for r in rows.values()), "in", oracle_pool.workers(), "workers")
    # only the listed rows leave the GPU (the 128K output is 17 GB)
    sel = {b: torch.tensor(rr, dtype=torch.long, device="cuda") for b, rr in rows.items()}
    g_idx = {b: idx[b].index_select(0, t).cpu().numpy() for b, t in sel.items()}
    g_out = {b: out[b].index_select(0, t).cpu().numpy().view(np.uint16) for b, t in sel.items()}
    g_lse = {b: lse[b].index_select(0, t).cpu().numpy() for b, t in sel.items()}
    del out, lse, idx
    res = oracle_pool.check_rows(wl, rows, g_idx, g_out, g_lse)
    s = oracle_pool.summarise(res)
    _say(name, "full size:", s)
    assert not s["failed"], s["failed"][:5]
    assert s["compared"] == s["rows"] == sum(len(r) for r in rows.values())
    assert s["normwise_max"] <= ATTN_MAX_REL and s["lse_max"] <= LSE_ABS


@pytest.mark.timeout(300)
@pytest.mark.parametrize("q_pos0", [98304, 130560])
def test_indexer_p128k_chunk_rel_rms(q_pos0):
    """A 512-row chunk of the 128K prefill as dsa_forward launches it (long
    key blocks at these positions), every row against the oracle."""
    full = W.WORKLOADS["p128k"]
    T = 512
    wl = W.custom("p128k", n_q=T, q_pos0=q_pos0)
    d = SD.fill_inputs(full)
    dims = dsa.Dims.of(wl)
    sc = torch.full((1, T, full.n_kv), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores(dims, d["q_idx"][:, q_pos0:], d["q_scale"][:, q_pos0:], d["w_idx"][:, q_pos0:],
                           d["k_idx"], d["k_scale"], sc, full.n_kv)
    torch.cuda.synchronize()
    del d
    scn = sc.cpu().numpy()
    hs = HostSide(full)
    pairs = []
    for i in range(T):
        n = q_pos0 + i + 1
        assert not np.any(np.isnan(scn[0, i, :n])) and np.all(np.isnan(scn[0, i, n:])), i
        pairs.append((scn[0, i, :n], hs.scores(q_pos0 + i)))
    err = score_rel_rms(pairs)
    _say("p128k chunk at", q_pos0, "indexer rel RMS", err)
    assert err <= SCORE_REL_RMS
