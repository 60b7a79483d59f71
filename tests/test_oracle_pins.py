"""Pins of the CPU reference (oracle/) to things other than itself:
hand-worked examples from the definitions (tests/golden), closed forms,
library routines for special cases, and invariants the method guarantees.
A plausible slip in the reference (dropped ReLU, ReLU after the head sum, a
wrong weight/head pairing, a wrong sign, a transposed operand, an off-by-one
in the causal window, the wrong tie order, a softmax over the wrong set)
fails at least one of these."""
import math

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O


def _parse_floats(s):
    return [float(x) for x in s.replace("|", " ").split()]


# ------------------------------------------------------------------ FP8 / bf16 decode
def test_e4m3_spot_values_from_ocp_spec(golden_dir):
    for line in open(f"{golden_dir}/e4m3_spot.txt"):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = O.e4m3_decode(np.uint8(int(code, 16)))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), (code, got, val)
            if val == "-0":
                assert np.signbit(got)


def test_e4m3_all_codes_match_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_decode(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.isnan(got).sum() == 2  # only S.1111.111


def test_bf16_decode_matches_torch():
    bits = np.random.RandomState(0).randint(0, 1 << 16, size=4096).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite values
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_decode(bits), ref)


# ------------------------------------------------------------------ indexer, Eq. (1)
def _indexer_golden(golden_dir):
    keys, queries, topk = [], {}, None
    for line in open(f"{golden_dir}/indexer_worked.txt"):
        if line.startswith("#") or not line.strip():
            continue
        if line.startswith("key"):
            keys.append(_parse_floats(line.split(":")[1]))
        elif line.startswith("query"):
            head, rest = line.split("heads:")
            name, p = head.split()[0], int(head.split("p=")[1])
            hs, rest = rest.split("weights:")
            ws, sc = rest.split("scores:")
            heads = [_parse_floats(h) for h in hs.split("|") if h.strip()]
            queries[name] = (p, np.array(heads), np.array(_parse_floats(ws)), np.array(_parse_floats(sc)))
        elif line.startswith("topk"):
            k = int(line.split("k=")[1].split(":")[0])
            topk = (k, [int(x) for x in line.split(":")[1].split()])
    return np.array(keys), queries, topk


def test_indexer_worked_example(golden_dir):
    keys, queries, _ = _indexer_golden(golden_dir)
    for name, (p, q, w, want) in queries.items():
        got = O.indexer_row(q, w, keys, p)
        assert got.shape == (p + 1,), name
        assert np.array_equal(got, want.astype(np.float32)), (name, got, want)


def test_topk_of_worked_indexer_row(golden_dir):
    keys, queries, (k, want) = _indexer_golden(golden_dir)
    p, q, w, _ = queries["queryA"]
    sel = O.topk_row(O.indexer_row(q, w, keys, p), k)
    assert list(sel) == want


def test_indexer_single_head_unit_weight_is_relu_dot():
    # H_I = 1, w = 1: Eq. (1) reduces to ReLU(q . k) -- checked with torch.
    rs = np.random.RandomState(1)
    q = rs.randn(1, 16)
    k = rs.randn(40, 16)
    got = O.indexer_row(q, np.ones(1), k, 39)
    ref = torch.relu(torch.from_numpy(k) @ torch.from_numpy(q[0])).numpy().astype(np.float32)
    assert np.array_equal(got, ref)


def test_indexer_causal_window_and_cache_bound():
    rs = np.random.RandomState(2)
    q, w, k = rs.randn(4, 8), rs.randn(4), rs.randn(10, 8)
    assert O.indexer_row(q, w, k, 0).shape == (1,)       # a token sees itself
    assert O.indexer_row(q, w, k, 6).shape == (7,)
    assert O.indexer_row(q, w, k, 25).shape == (10,)     # capped by the cache length
    # entries do not depend on later keys
    k2 = k.copy(); k2[7:] = 1e6
    assert np.array_equal(O.indexer_row(q, w, k, 6), O.indexer_row(q, w, k2, 6))


def test_indexer_homogeneity_linearity_and_sign():
    rs = np.random.RandomState(3)
    q, k = rs.randn(6, 12), rs.randn(30, 12)
    w1, w2 = rs.randn(6), rs.randn(6)
    base = O.indexer_row(q, w1, k, 29).astype(np.float64)
    # positive scaling of q or of k scales the score (ReLU is positively homogeneous)
    assert np.allclose(O.indexer_row(2.5 * q, w1, k, 29), 2.5 * base, rtol=1e-6)
    assert np.allclose(O.indexer_row(q, w1, 0.25 * k, 29), 0.25 * base, rtol=1e-6)
    # linear in the head weights
    s12 = O.indexer_row(q, w1 + w2, k, 29).astype(np.float64)
    assert np.allclose(s12, base + O.indexer_row(q, w2, k, 29), rtol=1e-5, atol=1e-5)
    # non-negative weights give non-negative scores; flipping q and k together
    # leaves dot products and therefore scores unchanged
    assert np.all(O.indexer_row(q, np.abs(w1), k, 29) >= 0)
    assert np.array_equal(O.indexer_row(-q, w1, -k, 29), O.indexer_row(q, w1, k, 29))
    # orthogonal query and keys score zero
    qo = np.zeros((6, 12)); qo[:, 0] = 1
    ko = rs.randn(30, 12); ko[:, 0] = 0
    assert np.all(O.indexer_row(qo, w1, ko, 29) == 0)


def test_indexer_fp8_inputs_are_exact_in_float64():
    # With FP8 values, every product and partial sum of q.k is exact in
    # float64, so the score equals its value computed in exact rationals.
    from fractions import Fraction
    rs = np.random.RandomState(4)
    codes_q = rs.randint(0, 256, size=(2, 16)).astype(np.uint8)
    codes_k = rs.randint(0, 256, size=(3, 16)).astype(np.uint8)
    codes_q[(codes_q & 0x7F) == 0x7F] = 0
    codes_k[(codes_k & 0x7F) == 0x7F] = 0
    q = O.e4m3_decode(codes_q); k = O.e4m3_decode(codes_k)
    w = np.array([0.75, -1.25])
    got = O.indexer_row(q, w, k, 2)
    for s in range(3):
        exact = Fraction(0)
        for j in range(2):
            d = sum(Fraction(float(q[j, i])) * Fraction(float(k[s, i])) for i in range(16))
            exact += Fraction(float(w[j])) * max(d, Fraction(0))
        assert got[s] == np.float32(float(exact))


# ------------------------------------------------------------------ top-k
def test_topk_worked_examples(golden_dir):
    for line in open(f"{golden_dir}/topk_worked.txt"):
        if line.startswith("#") or not line.strip():
            continue
        k, sc, want = line.split("|")
        got = O.topk_row(np.array([float(x) for x in sc.split()], dtype=np.float32), int(k))
        assert list(got) == [int(x) for x in want.split()], line


@pytest.mark.parametrize("seed", range(5))
def test_topk_defining_properties_random_rows(seed):
    # Brute-force check of the definition: |S| = min(k, n); every chosen score
    # >= every unchosen score; among equal scores at the cutoff, the chosen
    # indices are the lowest ones; output sorted and padded.
    rs = np.random.RandomState(seed)
    n = rs.randint(1, 400)
    k = rs.randint(1, 300)
    x = np.round(rs.randn(n) * 3).astype(np.float32)   # many ties
    sel = O.topk_row(x, k)
    m = min(k, n)
    chosen = sel[:m]
    assert np.all(sel[m:] == -1)
    assert np.all(np.diff(chosen) > 0)
    rest = np.setdiff1d(np.arange(n), chosen)
    if rest.size:
        assert x[chosen].min() >= x[rest].max()
        tau = x[chosen].min()
        tied_out = rest[x[rest] == tau]
        tied_in = chosen[x[chosen] == tau]
        if tied_out.size:
            assert tied_in.max() < tied_out.min()


def test_topk_all_equal_and_short_rows():
    assert list(O.topk_row(np.zeros(50, np.float32), 7)) == list(range(7))
    assert list(O.topk_row(np.arange(5, dtype=np.float32), 8)) == [0, 1, 2, 3, 4, -1, -1, -1]


# ------------------------------------------------------------------ attention, Eq. (2)/(19)
def test_attention_single_entry_closed_form():
    rs = np.random.RandomState(5)
    q, kv = rs.randn(4, 10), rs.randn(6, 10)
    o, lse = O.sparse_mla_row(q, kv, np.array([3, -1, -1]), 0.3, 7)
    assert np.array_equal(o, np.broadcast_to(kv[3, :7], (4, 7)))
    assert np.allclose(lse, 0.3 * q @ kv[3], rtol=1e-14)


def test_attention_two_entries_sigmoid_closed_form():
    rs = np.random.RandomState(6)
    q, kv = rs.randn(3, 8), rs.randn(5, 8)
    o, lse = O.sparse_mla_row(q, kv, np.array([1, 4]), 0.7, 6)
    z1, z2 = 0.7 * q @ kv[1], 0.7 * q @ kv[4]
    a = 1.0 / (1.0 + np.exp(z2 - z1))
    assert np.allclose(o, a[:, None] * kv[1, :6] + (1 - a)[:, None] * kv[4, :6], rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, np.logaddexp(z1, z2), rtol=1e-12)


def test_attention_all_positions_equals_dense_causal_sdpa():
    # When k >= n_p the selection is every position, so the path is dense
    # causal MQA attention: checked against torch's SDPA in float64.
    rs = np.random.RandomState(7)
    L, H, Dk, Dv = 24, 4, 12, 8
    q, kv = rs.randn(L, H, Dk), rs.randn(L, Dk)
    scale = 1 / math.sqrt(Dk)
    got = np.stack([O.sparse_mla_row(q[t], kv, O.topk_row(np.zeros(t + 1, np.float32), 64), scale, Dv)[0]
                    for t in range(L)])
    qt = torch.from_numpy(q).permute(1, 0, 2)                          # [H, L, Dk]
    kt = torch.from_numpy(kv).unsqueeze(0).expand(H, L, Dk).contiguous()
    vt = torch.from_numpy(kv[:, :Dv]).unsqueeze(0).expand(H, L, Dv).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    assert np.allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_attention_softmax_weights_sum_to_one_and_lse_matches_logsumexp():
    from scipy.special import logsumexp
    rs = np.random.RandomState(8)
    q, kv = rs.randn(5, 16) * 3, rs.randn(100, 16)
    sel = np.array([0, 7, 9, 33, 50, 51, 99, -1, -1])
    o, lse, p = O.sparse_mla_row(q, kv, sel, 0.5, 16, return_weights=True)
    assert np.all(np.abs(p.sum(axis=1) - 1) < 1e-12)
    s = sel[sel >= 0]
    assert np.allclose(lse, logsumexp(0.5 * q @ kv[s].T, axis=1), rtol=1e-13)
    # the index scores never enter the weights: only the set matters, and its order does not
    perm = np.array([51, 99, 0, 33, 9, 7, 50])
    o2, lse2 = O.sparse_mla_row(q, kv, perm, 0.5, 16)
    assert np.allclose(o, o2, rtol=1e-12) and np.allclose(lse, lse2, rtol=1e-12)


def test_attention_eq20_mass_bound():
    # Sec. 5.2 Eq. (20): ||o_dense - o_sparse|| <= 2 (1 - M_k) V with M_k the
    # dense softmax mass on the selected set and V a bound on |v|.
    rs = np.random.RandomState(9)
    n, H, D = 200, 6, 16
    q, kv = rs.randn(H, D), rs.randn(n, D)
    dense, _, pd = O.sparse_mla_row(q, kv, np.arange(n), 0.4, D, return_weights=True)
    for k in (5, 50, 150):
        sel = rs.choice(n, size=k, replace=False)
        sparse, _ = O.sparse_mla_row(q, kv, sel, 0.4, D)
        mk = pd[:, sel].sum(axis=1)
        vmax = np.abs(kv).max()
        assert np.all(np.abs(dense - sparse).max(axis=1) <= 2 * (1 - mk) * vmax + 1e-12)


def test_whole_row_path_with_k_covering_row_is_dense():
    rs = np.random.RandomState(10)
    qI, wI, kI = rs.randn(4, 8), rs.randn(4), rs.randn(30, 8)
    q, kv = rs.randn(3, 12), rs.randn(30, 12)
    sc, sel, o, lse = O.dsa_row(qI, wI, kI, q, kv, 20, 32, 0.3, 10)
    assert list(sel[:21]) == list(range(21)) and np.all(sel[21:] == -1)
    od, _ = O.sparse_mla_row(q, kv, np.arange(21), 0.3, 10)
    assert np.array_equal(o, od)


# ------------------------------------------------------------------ cost figures (Sec. 1.1)
def test_cost_figures_of_the_pages():
    # 64 index heads x 128 dims = 8192 MAC per pair; 128 heads x (576 + 512)
    # = 139,264 MAC per selected pair, about 17x more; k = 2048 of 128K = 1.6%.
    assert 64 * 128 == 8192
    assert 128 * (576 + 512) == 139264
    assert round(139264 / 8192) == 17
    assert abs(2048 / 131072 - 0.016) < 0.0005


# ------------------------------------------------------------------ FP8 quantisation
def test_quantize_matches_torch_float8_and_the_input_generator():
    # The per-token quantiser against two independent implementations of the
    # same definition: torch's float8_e4m3fn conversion (round to nearest
    # even; every quotient here is at most 448 * (1 + 2^-23)) applied to the
    # scaled values, and the input generator's own encoder.
    from synth import gen
    rs = np.random.RandomState(11)
    x = (rs.randn(300, 128) * np.exp(rs.randn(300, 1) * 6)).astype(np.float32)
    x[0] = 0.0
    x[1, :] = -0.0
    x[2, 5] = -3e-7
    codes, scales = O.quantize_e4m3_tokens(x)
    assert scales[0] == 1.0 and np.all(codes[0] == 0) and np.all(codes[1] == 0x80)
    y = (x / scales[:, None]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    c2, s2 = gen.quantize_tokens_e4m3(x)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)


def test_quantize_ties_saturation_and_exact_values():
    # amax = 448 gives scale 1, so the codes are those of x itself.
    vals = O.E4M3_VALUES[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2                       # exact midpoints
    row = np.concatenate([[448.0], vals, mids, [-1.0625]]).astype(np.float32)
    pad = (-len(row)) % 4
    row = np.concatenate([row, np.zeros(pad, np.float32)])
    codes, scales = O.quantize_e4m3_tokens(row[None, :])
    assert scales[0] == 1.0
    c = codes[0]
    n = len(vals)
    assert np.array_equal(c[1:1 + n], np.arange(n, dtype=np.uint8))           # representable: exact
    tie = c[1 + n:1 + n + len(mids)]
    assert np.all(tie % 2 == 0) and np.all((tie == np.arange(len(mids))) | (tie == np.arange(1, len(mids) + 1)))
    assert c[1 + n + len(mids)] == (0x80 | 0x38)             # -1.0625 -> -1.0 (even mantissa)
    # A token whose amax / (amax / 448) rounds above 448 saturates to 0x7E.
    rs = np.random.RandomState(13)
    for _ in range(10000):
        amax = np.float32(rs.uniform(1, 100))
        sc = np.float32(amax / np.float32(448.0))
        if np.float32(amax / sc) > np.float32(448.0):
            break
    else:
        raise AssertionError("no rounding-up quotient found")
    codes, _ = O.quantize_e4m3_tokens(np.array([[amax, 0, 0, 0]], np.float32))
    assert codes[0, 0] == 0x7E


def test_quantize_round_trip_error_bound():
    # |decode(code) * scale - x| <= half a unit in the last place of the
    # E4M3 grid at |x / scale| (2^-10 * scale in the subnormal range).
    rs = np.random.RandomState(12)
    x = (rs.standard_cauchy((100, 64))).astype(np.float32)
    codes, scales = O.quantize_e4m3_tokens(x)
    back = O.e4m3_decode(codes) * scales[:, None].astype(np.float64)
    a = np.abs(x.astype(np.float64) / scales[:, None])
    ulp = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(np.abs(back - x) <= 0.5 * ulp * scales[:, None] * (1 + 1e-6) + 1e-30)


# ------------------------------------------------------------------ paged / variable-length caches
def test_gather_stats_worked_examples(golden_dir):
    for line in open(f"{golden_dir}/gather_stats_worked.txt"):
        if line.startswith("#") or not line.strip():
            continue
        ps, sel, want = (x.split() for x in line.split("|"))
        got = O.gather_stats([int(v) for v in sel], int(ps[0]))
        assert got == tuple(int(v) for v in want), (line, got)


def test_gather_stats_matches_a_walk_over_the_row():
    # An independent count: walk the ascending selection once, opening a run
    # whenever the index does not follow its predecessor and counting hits per
    # page in a dict.
    rs = np.random.RandomState(31)
    for _ in range(200):
        n = int(rs.randint(0, 3000))
        m = int(rs.randint(0, min(n, 300) + 1))
        sel = np.sort(rs.choice(n, size=m, replace=False)) if m else np.zeros(0, np.int64)
        ps = int(rs.choice([16, 64, 128]))
        runs, prev, hits = 0, None, {}
        for s in sel:
            if prev is None or s != prev + 1:
                runs += 1
            prev = s
            hits[s // ps] = hits.get(s // ps, 0) + 1
        want = (len(hits), runs, max(hits.values()) if hits else 0)
        padded = np.concatenate([sel, -np.ones(5, np.int64)])
        assert O.gather_stats(padded, ps) == want


def test_paged_gather_inverts_the_page_scatter():
    # Build a pool by scattering each sequence's pages to random slots; the
    # gather through the page table must give the dense tokens back, and an
    # identity table must be a plain slice.
    rs = np.random.RandomState(32)
    P, B, S = 16, 3, 80
    npages = (S + P - 1) // P
    dense = rs.randn(B, npages * P, 5)
    table = rs.permutation(B * npages + 4)[:B * npages].reshape(B, npages)
    pool = np.full((table.max() + 1) * P, np.nan)[:, None] * np.ones((1, 5))
    for b in range(B):
        for j in range(npages):
            pool[table[b, j] * P:(table[b, j] + 1) * P] = dense[b, j * P:(j + 1) * P]
    for b in range(B):
        n = int(rs.randint(1, S + 1))
        assert np.array_equal(O.paged_gather(pool, table[b], P, n), dense[b, :n])
    flat = dense.reshape(-1, 5)
    assert np.array_equal(O.paged_gather(flat, np.arange(npages) + npages, P, S), flat[npages * P:npages * P + S])


def test_varlen_rows_are_the_sequence_tail():
    # Decode sees itself as the last cached token; n_q new tokens are the last
    # n_q positions, and each row's candidate count is its position + 1.
    assert O.varlen_positions(100, 1) == [99]
    assert O.varlen_positions(7, 3) == [4, 5, 6]
    for L, n_q in ((5, 5), (130, 4)):
        pos = O.varlen_positions(L, n_q)
        assert [O.n_candidates(p, L) for p in pos] == list(range(L - n_q + 1, L + 1))


# ------------------------------------------------------------------ indexer KL (Eq. (4))
def test_indexer_kl_is_zero_when_the_indexer_matches_the_attention():
    # One head: p is that head's softmax over the set.  Index scores equal to
    # the head's logits (up to a constant) give softmax(I) = p, so KL = 0;
    # any other scores give KL > 0 (Gibbs' inequality).
    rs = np.random.RandomState(51)
    S, Dk, Dv, sc = 40, 12, 8, 0.3
    q = rs.randn(1, Dk)
    kv = rs.randn(S, Dk)
    sel = np.array([1, 4, 9, 17, 30, 33, -1, -1])
    logits = sc * (kv @ q[0])
    assert abs(O.indexer_kl_row(q, kv, sel, logits + 7.5, sc, Dv)) < 1e-12
    other = logits + rs.randn(S) * 0.5
    assert O.indexer_kl_row(q, kv, sel, other, sc, Dv) > 1e-4


def test_indexer_kl_closed_form_two_entries():
    # Two selected tokens, H heads with logit gaps d_h: p_1 = mean_h sigmoid(d_h)
    # (head weights summed then L1-normalised), q_1 = sigmoid(I_1 - I_0);
    # KL = p0 ln(p0/q0) + p1 ln(p1/q1).
    rs = np.random.RandomState(52)
    H, Dk, sc = 3, 6, 0.7
    q = rs.randn(H, Dk)
    kv = rs.randn(2, Dk)
    d = sc * (q @ (kv[1] - kv[0]))
    p1 = np.mean(1.0 / (1.0 + np.exp(-d)))
    I = np.array([0.2, -1.1])
    q1 = 1.0 / (1.0 + np.exp(-(I[1] - I[0])))
    want = (1 - p1) * np.log((1 - p1) / (1 - q1)) + p1 * np.log(p1 / q1)
    assert abs(O.indexer_kl_row(q, kv, np.array([0, 1]), I, sc, 4) - want) < 1e-12


def test_indexer_kl_ignores_padding_and_order_and_empty_rows():
    rs = np.random.RandomState(53)
    q, kv, I = rs.randn(4, 10), rs.randn(30, 10), rs.randn(30)
    a = O.indexer_kl_row(q, kv, np.array([3, 7, 12, 20, -1]), I, 0.4, 6)
    b = O.indexer_kl_row(q, kv, np.array([20, -1, 12, 3, 7]), I, 0.4, 6)
    assert abs(a - b) < 1e-12 and a > 0
    assert O.indexer_kl_row(q, kv, np.array([-1, -1]), I, 0.4, 6) == 0.0


# ----------------------------------------------------------------- masked MHA mode
def _mha_case(rs, H=3, dn=5, dr=3, dim_v=7, dvh=4, S=20):
    kv = rs.randn(S, dim_v + dr)
    return kv, rs.randn(H, dn, dim_v), rs.randn(H, dvh, dim_v), rs.randn(H, dn + dr)


def test_masked_mha_equals_mqa_attention_with_absorbed_query():
    # Fig. 7 discussion of the analysis page: MHA mode (decompressed per-head
    # keys/values) and MQA mode (decompression folded into the query) are the
    # same attention.  MQA form: q_abs[h] = [W_UK[h]^T q_nope[h] | q_rope[h]]
    # over the latent rows, then W_UV[h] applied to the latent-space output.
    # Rectangular dims catch a transposed decompression matrix.
    rs = np.random.RandomState(40)
    kv, wuk, wuv, _ = _mha_case(rs)
    dn = wuk.shape[1]
    for p, sel in ((15, [1, 4, 7, 9, 15, -1, -1]), (6, [0, 1, 2, 3, 4, 5, 6]), (19, [19]), (3, [2, -1])):
        q = rs.randn(3, dn + 3)
        o, lse = O.masked_mha_row(q, kv, wuk, wuv, np.array(sel), p, 0.3, 7)
        q_abs = np.concatenate([np.einsum("hdc,hd->hc", wuk, q[:, :dn]), q[:, dn:]], axis=1)
        o_lat, lse_lat = O.sparse_mla_row(q_abs, kv, np.array(sel), 0.3, 7)
        assert np.allclose(o, np.einsum("hdc,hc->hd", wuv, o_lat), rtol=1e-12, atol=1e-12)
        assert np.allclose(lse, lse_lat, rtol=1e-13)


def test_masked_mha_with_every_key_selected_is_dense_causal_sdpa():
    # Below the top-k size every causal key is selected, so masked MHA mode is
    # plain causal multi-head attention on the decompressed keys and values:
    # checked against torch's SDPA in float64.
    rs = np.random.RandomState(41)
    L, H, dn, dr, dim_v, dvh = 18, 4, 6, 2, 10, 5
    kv, wuk, wuv, _ = _mha_case(rs, H, dn, dr, dim_v, dvh, L)
    q = rs.randn(L, H, dn + dr)
    got = np.stack([O.masked_mha_row(q[t], kv, wuk, wuv, np.arange(t + 1), t, 0.4, dim_v)[0] for t in range(L)])
    k = np.concatenate([np.einsum("hdc,sc->hsd", wuk, kv[:, :dim_v]),
                        np.broadcast_to(kv[None, :, dim_v:], (H, L, dr))], axis=2)
    v = np.einsum("hdc,sc->hsd", wuv, kv[:, :dim_v])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2).contiguous(), torch.from_numpy(k.copy()), torch.from_numpy(v),
        is_causal=True, scale=0.4)
    assert np.allclose(got, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_masked_mha_mask_is_a_boolean_sdpa_mask_and_drops_future_keys():
    # The selection acts as a boolean attention mask over the causal keys;
    # entries past the row's position or padding change nothing.
    rs = np.random.RandomState(42)
    L, H, dn, dr, dim_v, dvh = 16, 2, 4, 4, 8, 4
    kv, wuk, wuv, _ = _mha_case(rs, H, dn, dr, dim_v, dvh, L)
    q = rs.randn(L, H, dn + dr)
    allowed = np.zeros((L, L), dtype=bool)
    got = []
    for t in range(L):
        sel = np.sort(rs.choice(t + 1, size=min(t + 1, 5), replace=False))
        allowed[t, sel] = True
        noisy = np.concatenate([sel, [t + 1 + j for j in range(2) if t + 1 + j < L], [-1, -1]])
        got.append(O.masked_mha_row(q[t], kv, wuk, wuv, noisy, t, 0.5, dim_v))
    k = np.concatenate([np.einsum("hdc,sc->hsd", wuk, kv[:, :dim_v]),
                        np.broadcast_to(kv[None, :, dim_v:], (H, L, dr))], axis=2)
    v = np.einsum("hdc,sc->hsd", wuv, kv[:, :dim_v])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2).contiguous(), torch.from_numpy(k.copy()), torch.from_numpy(v),
        attn_mask=torch.from_numpy(allowed), scale=0.5)
    assert np.allclose(np.stack([g[0] for g in got]), ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_masked_mha_single_key_and_empty_rows():
    rs = np.random.RandomState(43)
    kv, wuk, wuv, q = _mha_case(rs)
    o, lse = O.masked_mha_row(q, kv, wuk, wuv, np.array([6, -1]), 9, 0.3, 7)
    assert np.allclose(o, wuv @ kv[6, :7], rtol=1e-13)
    z = 0.3 * (np.einsum("hd,hd->h", q[:, :5], wuk @ kv[6, :7]) + q[:, 5:] @ kv[6, 7:])
    assert np.allclose(lse, z, rtol=1e-13)
    o, lse = O.masked_mha_row(q, kv, wuk, wuv, np.array([12, -1]), 9, 0.3, 7)   # only a future key
    assert np.array_equal(o, np.zeros_like(o)) and np.all(lse == -np.inf)


def test_mha_decompress_worked_example():
    # MHA mode (the analysis page, Fig. 7 discussion): per-head keys
    # k_nope[h, s] = W_UK[h] c_s and values v[h, s] = W_UV[h] c_s over the
    # first dim_v latent dims; the remaining dims are the shared rope part.
    # Worked by hand on two latent rows, dim_v = 3, rope 2, two heads;
    # rectangular W (2 x 3 and 1 x 3) so a transposed matrix cannot pass.
    kv = np.array([[1.0, 2.0, 3.0, 10.0, 20.0],
                   [4.0, 5.0, 6.0, 30.0, 40.0]])
    w_uk = np.array([[[1.0, 0.0, 0.0], [0.0, 0.0, 2.0]],
                     [[0.0, 1.0, 0.0], [1.0, 1.0, 1.0]]])
    w_uv = np.array([[[0.0, 1.0, 0.0]],
                     [[1.0, 0.0, -1.0]]])
    k_nope, v, rope = O.mha_decompress(kv, w_uk, w_uv, 3)
    assert k_nope.shape == (2, 2, 2) and v.shape == (2, 2, 1) and rope.shape == (2, 2)
    assert np.array_equal(k_nope[0], [[1.0, 6.0], [4.0, 12.0]])     # [c0, 2 c2]
    assert np.array_equal(k_nope[1], [[2.0, 6.0], [5.0, 15.0]])     # [c1, c0 + c1 + c2]
    assert np.array_equal(v[0], [[2.0], [5.0]])                     # c1
    assert np.array_equal(v[1], [[-2.0], [-2.0]])                   # c0 - c2
    assert np.array_equal(rope, [[10.0, 20.0], [30.0, 40.0]])


def test_candidate_and_selection_counts():
    # n_p = min(p + 1, S) causal candidates; m_p = min(k, n_p) selected
    # (Sec. 5.1 of the analysis page: a short row keeps everything it has).
    assert [O.n_candidates(p, 10) for p in (0, 4, 9, 12)] == [1, 5, 10, 10]
    assert [O.n_selected(p, 10, 4) for p in (0, 2, 3, 9)] == [1, 3, 4, 4]
    assert O.n_selected(9, 10, 16) == 10


def test_selection_mask_bits():
    m = O.selection_mask(np.array([0, 3, 3, 31, 32, -1, 40, 7]), 33)
    assert np.flatnonzero(m).tolist() == [0, 3, 7, 31, 32]


# ----------------------------------------------------------------- dequantisation and cache append
def test_dequant_scale_multiplies_each_token():
    """One scale per token: the scale of token t multiplies every value of
    token t (and nothing of another token), for 2-D and 3-D code arrays.
    Codes from the OCP E4M3 table: 0x38 = 1, 0x40 = 2, 0xB8 = -1, 0x30 = 0.5."""
    codes = np.array([[0x38, 0x40, 0xB8], [0x38, 0x40, 0xB8]], np.uint8)   # 2 tokens x 3 values
    got = O.dequant_e4m3(codes, np.array([2.0, 0.5], np.float32))
    assert np.array_equal(got, [[2.0, 4.0, -2.0], [0.5, 1.0, -0.5]])
    codes3 = np.array([[[0x38, 0x30], [0x40, 0x38]], [[0xB8, 0x40], [0x30, 0x30]]], np.uint8)   # [B=2, T=2, d=2]
    scales3 = np.array([[1.0, 2.0], [4.0, 8.0]], np.float32)
    want3 = np.array([[[1.0, 0.5], [4.0, 2.0]], [[-4.0, 8.0], [4.0, 4.0]]])
    assert np.array_equal(O.dequant_e4m3(codes3, scales3), want3)


def _cache_append_golden(golden_dir):
    rows = []
    for line in open(f"{golden_dir}/cache_append_worked.txt"):
        line = line.split("#")[0].strip()
        if not line:
            continue
        lhs, sc, codes = (x.strip() for x in line.split("|"))
        f = lhs.split()
        rows.append((int(f[0]), int(f[1]), [float(v) for v in f[2:]], float(sc), [int(c, 16) for c in codes.split()]))
    return rows


def test_cache_append_worked_example(golden_dir):
    """Rows pos0 .. pos0 + n - 1 of every sequence receive the new tokens'
    codes, scales and latents; every other row keeps its old contents."""
    B, S, d, pos0, n = 2, 5, 4, 2, 2
    gold = _cache_append_golden(golden_dir)
    k_new = np.zeros((B, n, d), np.float32)
    for b, t, x, _, _ in gold:
        k_new[b, t] = x
    kv_new = np.arange(B * n * 3, dtype=np.float64).reshape(B, n, 3) + 100.0
    kc0 = np.full((B, S, d), 0x11, np.uint8)
    ks0 = np.full((B, S), 3.0, np.float32)
    kv0 = np.full((B, S, 3), 9.0)
    kc, ks, kv = O.cache_append(kc0, ks0, kv0, k_new, kv_new, pos0)
    for b, t, _, scale, codes in gold:
        assert np.array_equal(kc[b, pos0 + t], codes), (b, t)
        assert ks[b, pos0 + t] == np.float32(scale), (b, t)
        assert np.array_equal(kv[b, pos0 + t], kv_new[b, t])
    other = [r for r in range(S) if not pos0 <= r < pos0 + n]
    assert np.all(kc[:, other] == 0x11) and np.all(ks[:, other] == 3.0) and np.all(kv[:, other] == 9.0)
    # the inputs are not modified, and the codes are those of the quantiser
    assert np.all(kc0 == 0x11) and np.all(ks0 == 3.0) and np.all(kv0 == 9.0)
    codes_q, scales_q = O.quantize_e4m3_tokens(k_new)
    assert np.array_equal(kc[:, pos0:pos0 + n], codes_q) and np.array_equal(ks[:, pos0:pos0 + n], scales_q)
    # without latents only the key caches change
    kc2, ks2, kv2 = O.cache_append(kc0, ks0, None, k_new, None, pos0)
    assert kv2 is None and np.array_equal(kc2, kc) and np.array_equal(ks2, ks)
