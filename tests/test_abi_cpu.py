"""The C ABI library loads without a GPU, exports every symbol include/dsa.h
declares, and rejects invalid calls on the host before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_attention_long_amd as dsa
from sparse_attention_long_amd.dsa import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = dsa.lib()
    declared = _header_functions()
    assert len(declared) >= 9
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(dsa.EXPORTS)


def test_version_and_status_strings():
    assert dsa.dsa_version() == 200
    L = dsa.lib()
    assert L.dsa_status_string(0) == b"ok"
    assert L.dsa_status_string(3) == b"workspace too small"


def _dims(**kw):
    base = dict(batch=1, n_q=8, n_kv=8, q_pos0=0, idx_heads=64, idx_dim=128, heads=128, dim_qk=576, dim_v=512, topk=4)
    base.update(kw)
    return Dims(**base)


FAKE = 1 << 20   # an aligned, never-dereferenced address: validation fails before any use


@pytest.mark.parametrize("kw,status", [
    (dict(n_q=0), dsa.dsa.ERR_INVALID_ARG),
    (dict(q_pos0=-1), dsa.dsa.ERR_INVALID_ARG),
    (dict(q_pos0=1), dsa.dsa.ERR_INVALID_ARG),           # positions beyond the cache
    (dict(topk=0), dsa.dsa.ERR_UNSUPPORTED),
    (dict(topk=2049), dsa.dsa.ERR_UNSUPPORTED),
    (dict(idx_heads=65), dsa.dsa.ERR_UNSUPPORTED),
    (dict(idx_dim=100), dsa.dsa.ERR_UNSUPPORTED),
])
def test_indexer_validation(kw, status):
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_indexer_scores(_dims(**kw), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, stream=0)
    assert e.value.status == status


def test_indexer_rejects_small_ld_null_and_misaligned():
    for args, ld in (((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 7), ((FAKE, FAKE, FAKE, 0, FAKE, FAKE), 8),
                     ((FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE), 8)):
        with pytest.raises(dsa.DSAError) as e:
            dsa.dsa_indexer_scores(_dims(), *args, ld, stream=0)
        assert e.value.status == dsa.dsa.ERR_INVALID_ARG


def test_topk_validation():
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_topk(_dims(n_kv=300000, n_q=1, q_pos0=0), FAKE, 300000, FAKE, stream=0)
    assert e.value.status == dsa.dsa.ERR_UNSUPPORTED
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_topk(_dims(), FAKE, 4, FAKE, stream=0)
    assert e.value.status == dsa.dsa.ERR_INVALID_ARG


def test_attention_validation_and_workspace():
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_sparse_mla_attn(_dims(dim_qk=128, dim_v=64), FAKE, FAKE, FAKE, 0.1, FAKE, stream=0)
    assert e.value.status == dsa.dsa.ERR_UNSUPPORTED
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(dsa.DSAError) as e:
            dsa.dsa_sparse_mla_attn(_dims(), FAKE, FAKE, FAKE, bad, FAKE, stream=0)
        assert e.value.status == dsa.dsa.ERR_INVALID_ARG
    # decode-like shapes split the selected set and need a workspace
    d = _dims(batch=64, n_q=1, n_kv=131072, q_pos0=131071, topk=2048)
    need = dsa.dsa_attn_workspace_size(d)
    assert need == 64 * 4 * 128 * (512 * 2 + 4)   # bf16 partial outputs + f32 log-sum-exp
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_sparse_mla_attn(d, FAKE, FAKE, FAKE, 0.1, FAKE, ws=FAKE, ws_bytes=need - 1, stream=0)
    assert e.value.status == dsa.dsa.ERR_WORKSPACE
    # many rows: no split, no workspace
    assert dsa.dsa_attn_workspace_size(_dims(n_q=4096, n_kv=4096, topk=2048)) == 0
    # one sequence's latent cache must stay below 4 GiB (32-bit row offsets)
    limit = (1 << 32) // (576 * 2)                       # 3,728,270 rows of 1152 B
    assert dsa.dsa_attn_workspace_size(_dims(n_q=1, n_kv=limit, q_pos0=limit - 1, topk=2048)) > 0
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_sparse_mla_attn(_dims(n_q=1, n_kv=limit + 1, q_pos0=limit, topk=2048), FAKE, FAKE, FAKE, 0.1, FAKE,
                                ws=FAKE, ws_bytes=1 << 30, stream=0)
    assert e.value.status == dsa.dsa.ERR_UNSUPPORTED and "4 GiB" in str(e.value)
    # the workspace does not depend on the cache layout (page pools have no such limit)
    assert dsa.dsa_attn_workspace_size(_dims(n_q=1, n_kv=limit + 1, q_pos0=limit, topk=2048)) > 0


def test_forward_workspace_plan():
    d = _dims(n_q=131072, n_kv=131072, topk=2048)
    ws = dsa.dsa_forward_workspace_size(d)
    # one 512-row chunk: 256 MiB of scores plus 4 MiB of indices
    assert ws == 512 * 131072 * 4 + 512 * 2048 * 4
    plan = dsa.dsa.dsa_forward_plan_of(d)
    assert (plan.chunk_rows, plan.topk_parts, plan.attn_splits, plan.workspace_bytes) == (512, 1, 1, ws)
    # fewer rows than a chunk: the chunk shrinks to them
    one = _dims(n_q=256, n_kv=131072, q_pos0=131072 - 256, topk=2048)
    assert dsa.dsa_forward_workspace_size(one) == 256 * 131072 * 4 + 256 * 2048 * 4
    # a decode step (64 sequences, one row each) is one chunk with scores,
    # indices, 4-way split attention partials and the top-k part lists
    dec = _dims(batch=64, n_q=1, n_kv=131072, q_pos0=131071, topk=2048)
    partials = 64 * 4 * 128 * (512 * 2 + 4)
    base = 64 * 131072 * 4 + 64 * 2048 * 4 + partials
    assert base <= dsa.dsa_forward_workspace_size(dec) < 2 * base
    plan = dsa.dsa.dsa_forward_plan_of(dec)
    assert (plan.chunk_rows, plan.topk_parts, plan.attn_splits) == (1, 4, 4)
    assert plan.workspace_bytes == dsa.dsa_forward_workspace_size(dec)
    # the standalone top-k with a workspace splits the same way
    assert dsa.dsa.dsa_topk_workspace_size(dec) == dsa.dsa_forward_workspace_size(dec) - base
    assert dsa.dsa.dsa_topk_workspace_size(d) == 0
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa.dsa_topk_ws(dec, FAKE, 131072, FAKE, ws=FAKE, ws_bytes=dsa.dsa.dsa_topk_workspace_size(dec) - 1,
                            stream=0)
    assert e.value.status == dsa.dsa.ERR_WORKSPACE
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa.dsa_forward_plan_of(_dims(heads=7, dim_qk=100))   # dim_v 512 > dim_qk 100
    assert e.value.status == dsa.dsa.ERR_INVALID_ARG
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_forward(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.07, FAKE, ws=FAKE, ws_bytes=ws - 1, stream=0)
    assert e.value.status == dsa.dsa.ERR_WORKSPACE
    assert dsa.dsa_forward_workspace_size(_dims(heads=7, dim_qk=100)) == 0   # unsupported dims


def test_quantize_validation():
    for args, status in (((FAKE, 2, 4, 128), dsa.dsa.ERR_INVALID_ARG),      # bad dtype
                         ((FAKE, 0, 4, 130), dsa.dsa.ERR_UNSUPPORTED),      # length not a multiple of 4
                         ((FAKE, 0, 4, 20000), dsa.dsa.ERR_UNSUPPORTED),    # too long
                         ((FAKE + 8, 0, 4, 128), dsa.dsa.ERR_INVALID_ARG),  # f32 input not 16-byte aligned
                         ((0, 0, 4, 128), dsa.dsa.ERR_INVALID_ARG)):        # null
        x, dt, n, L = args
        with pytest.raises(dsa.DSAError) as e:
            dsa.dsa.dsa_quantize_e4m3(x, n, L, FAKE, FAKE, dtype=dt, stream=0)
        assert e.value.status == status


def test_cache_append_validation():
    with pytest.raises(dsa.DSAError) as e:   # new positions past the cache
        dsa.dsa.dsa_cache_append(_dims(n_q=2, n_kv=8, q_pos0=7), FAKE, FAKE, FAKE, k_dtype=0, stream=0)
    assert e.value.status == dsa.dsa.ERR_INVALID_ARG
    with pytest.raises(dsa.DSAError) as e:   # latent source without a latent cache
        dsa.dsa.dsa_cache_append(_dims(n_q=1, n_kv=8, q_pos0=7), FAKE, FAKE, FAKE, kv_new=FAKE, k_dtype=0, stream=0)
    assert e.value.status == dsa.dsa.ERR_INVALID_ARG
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa.dsa_cache_append(_dims(n_q=1, n_kv=8, q_pos0=7, idx_dim=6), FAKE, FAKE, FAKE, k_dtype=1, stream=0)
    assert e.value.status == dsa.dsa.ERR_UNSUPPORTED


def _layout(**kw):
    base = dict(seq_lens=FAKE, page_table=FAKE + 4096, page_size=64, max_pages=4, num_pages=16)
    base.update(kw)
    return dsa.dsa.PagedKV.of(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(seq_lens=None), dsa.dsa.ERR_INVALID_ARG),
    (dict(seq_lens=FAKE + 2), dsa.dsa.ERR_INVALID_ARG),          # misaligned
    (dict(page_size=32), dsa.dsa.ERR_UNSUPPORTED),               # not a multiple of 64
    (dict(page_size=0), dsa.dsa.ERR_UNSUPPORTED),
    (dict(max_pages=1), dsa.dsa.ERR_INVALID_ARG),                # 1 x 64 < n_kv = 200
    (dict(num_pages=0), dsa.dsa.ERR_UNSUPPORTED),
    (dict(num_pages=1 << 25, page_size=64), dsa.dsa.ERR_UNSUPPORTED),   # pool of 2^31 rows
])
def test_paged_layout_validation(kw, status):
    d = _dims(batch=2, n_q=1, n_kv=200, topk=16)
    lay = _layout(**kw)
    for call in (lambda: dsa.dsa.dsa_indexer_scores_paged(d, lay, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 200, stream=0),
                 lambda: dsa.dsa.dsa_topk_paged(d, lay, FAKE, 200, FAKE, stream=0),
                 lambda: dsa.dsa.dsa_sparse_mla_attn_paged(d, lay, FAKE, FAKE, FAKE, 0.1, FAKE, ws=FAKE,
                                                           ws_bytes=1 << 30, stream=0),
                 lambda: dsa.dsa.dsa_forward_paged(d, lay, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE,
                                                   ws=FAKE, ws_bytes=1 << 30, stream=0)):
        with pytest.raises(dsa.DSAError) as e:
            call()
        assert e.value.status == status


def test_paged_calls_keep_the_other_checks():
    d = _dims(batch=2, n_q=1, n_kv=200, topk=16)
    with pytest.raises(dsa.DSAError) as e:   # ld below n_kv
        dsa.dsa.dsa_indexer_scores_paged(d, _layout(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 199, stream=0)
    assert e.value.status == dsa.dsa.ERR_INVALID_ARG
    with pytest.raises(dsa.DSAError) as e:   # forward workspace too small
        dsa.dsa.dsa_forward_paged(d, _layout(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE,
                                  ws=FAKE, ws_bytes=16, stream=0)
    assert e.value.status == dsa.dsa.ERR_WORKSPACE
    # q_pos0 plays no part in the paged calls (positions come from seq_lens)
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa.dsa_topk_paged(_dims(batch=2, n_q=1, n_kv=200, topk=16, q_pos0=5000), _layout(), FAKE, 199, FAKE,
                               stream=0)
    assert e.value.status == dsa.dsa.ERR_INVALID_ARG and "ld" in str(e.value)


def test_gather_stats_validation():
    for kw, ps, status in ((dict(), 0, dsa.dsa.ERR_INVALID_ARG), (dict(topk=4096), 64, dsa.dsa.ERR_UNSUPPORTED),
                           (dict(n_q=0), 64, dsa.dsa.ERR_INVALID_ARG)):
        with pytest.raises(dsa.DSAError) as e:
            dsa.dsa.dsa_gather_stats(_dims(**kw), ps, FAKE, FAKE, stream=0)
        assert e.value.status == status


def test_indexer_kl_validation():
    d = _dims(batch=2, n_q=1, n_kv=200, topk=16)
    for kw, status in ((dict(lse=None), dsa.dsa.ERR_INVALID_ARG), (dict(ld=100), dsa.dsa.ERR_INVALID_ARG),
                       (dict(kl=FAKE + 2), dsa.dsa.ERR_INVALID_ARG), (dict(sm=0.0), dsa.dsa.ERR_INVALID_ARG)):
        a = dict(lse=FAKE, ld=200, kl=FAKE, sm=0.1)
        a.update(kw)
        with pytest.raises(dsa.DSAError) as e:
            dsa.dsa.dsa_indexer_kl(d, None, FAKE, FAKE, FAKE, a["lse"], FAKE, a["ld"], a["sm"], a["kl"], stream=0)
        assert e.value.status == status
    with pytest.raises(dsa.DSAError) as e:   # a paged layout is checked as in the _paged calls
        dsa.dsa.dsa_indexer_kl(d, _layout(page_size=32), FAKE, FAKE, FAKE, FAKE, FAKE, 200, 0.1, FAKE, stream=0)
    assert e.value.status == dsa.dsa.ERR_UNSUPPORTED
    with pytest.raises(dsa.DSAError) as e:   # the training forward needs kl and lse
        dsa.dsa.dsa_forward_kl(d, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, None, FAKE,
                               ws=FAKE, ws_bytes=1 << 30, stream=0)
    assert e.value.status == dsa.dsa.ERR_INVALID_ARG


def test_masked_mha_validation():
    D = dsa.dsa
    d = _dims(n_q=64, n_kv=64, topk=16)
    # unsupported per-head dims, too few rope dims, too long a cache
    for dd, dn, dvh in ((d, 64, 128), (d, 128, 64), (_dims(n_q=64, n_kv=64, dim_qk=512, dim_v=512), 128, 128),
                        (_dims(n_q=1, n_kv=70000, q_pos0=69999), 128, 128)):
        with pytest.raises(dsa.DSAError) as e:
            D.dsa_masked_mha_attn(dd, dn, dvh, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, stream=0)
        assert e.value.status in (D.ERR_UNSUPPORTED, D.ERR_INVALID_ARG)
        assert D.dsa_masked_mha_workspace_size(dd, dn, dvh) == 0
    # bad scale, misaligned output, null mask
    for args in ((FAKE, FAKE, 0.0, FAKE), (FAKE, FAKE, 0.1, FAKE + 8), (FAKE, None, 0.1, FAKE)):
        with pytest.raises(dsa.DSAError) as e:
            D.dsa_masked_mha_attn(d, 128, 128, args[0], FAKE, FAKE, FAKE, args[1], args[2], args[3], stream=0)
        assert e.value.status == D.ERR_INVALID_ARG
    with pytest.raises(dsa.DSAError) as e:
        D.dsa_mha_decompress(d, 128, 128, FAKE, FAKE, FAKE, 65, FAKE, FAKE, stream=0)   # n_rows > n_kv
    assert e.value.status == D.ERR_INVALID_ARG
    with pytest.raises(dsa.DSAError) as e:
        D.dsa_selection_mask(_dims(n_q=1, n_kv=70000, q_pos0=69999), FAKE, FAKE, stream=0)
    assert e.value.status == D.ERR_UNSUPPORTED


def test_masked_mha_workspace_plan():
    D = dsa.dsa
    d = _dims(n_q=4096, n_kv=4096, topk=2048)
    ws = D.dsa_masked_mha_workspace_size(d, 128, 128)
    # scores + indices of one 4096-row chunk, the bitmap, and per-head K and V of the 4096 visible rows
    assert ws == 4096 * 4096 * 4 + 4096 * 2048 * 4 + 128 * 4096 * 4 + 2 * 128 * 4096 * 128 * 2
    with pytest.raises(dsa.DSAError) as e:
        D.dsa_masked_mha_forward(d, 128, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.07, FAKE,
                                 ws=FAKE, ws_bytes=ws - 1, stream=0)
    assert e.value.status == D.ERR_WORKSPACE


def test_validate_host_checks():
    D = dsa.dsa
    d = _dims(batch=2, n_q=1, n_kv=200, topk=16)
    for kw, status in ((dict(counts=None), D.ERR_INVALID_ARG), (dict(counts=FAKE + 2), D.ERR_INVALID_ARG),
                       (dict(q_scale=FAKE + 2), D.ERR_INVALID_ARG), (dict(idx=FAKE + 1), D.ERR_INVALID_ARG)):
        a = dict(q_scale=FAKE, w_idx=FAKE, k_scale=FAKE, idx=FAKE, counts=FAKE)
        a.update(kw)
        with pytest.raises(dsa.DSAError) as e:
            D.dsa_validate(d, None, a["q_scale"], a["w_idx"], a["k_scale"], a["idx"], a["counts"], stream=0)
        assert e.value.status == status
    with pytest.raises(dsa.DSAError) as e:   # the dims are checked as in the other calls
        D.dsa_validate(_dims(q_pos0=1), None, FAKE, None, None, None, FAKE, stream=0)
    assert e.value.status == D.ERR_INVALID_ARG
    with pytest.raises(dsa.DSAError) as e:   # and a paged layout as in the _paged calls
        D.dsa_validate(d, _layout(page_size=32), FAKE, None, None, None, FAKE, stream=0)
    assert e.value.status == D.ERR_UNSUPPORTED
    assert len(D.VALIDATE_COUNTS) == 8


def test_topk_sample_indices_stay_inside_the_row():
    """The top-k kernel's sampled cutoff reads 32 blocks of 64 scores at
    e = floor(blk (n - 64) / 31) + j, j < 64, for rows of n >= 64 scores
    (shorter rows take no sample): every index lies in [0, n)."""
    for n in list(range(64, 5000)) + [131071, 131072, 262144]:
        blk = np.arange(32, dtype=np.int64)
        first = (blk * (n - 64)) // 31
        assert first.min() >= 0 and (first + 63).max() <= n - 1, n


def test_noalloc_attention_limit():
    D = dsa.dsa
    # 255 rows split two ways need 67 MB of partials: above the 40 MiB array
    d = _dims(batch=255, n_q=1, n_kv=131072, q_pos0=131071, topk=2048)
    assert dsa.dsa_attn_workspace_size(d) > 40 << 20
    with pytest.raises(dsa.DSAError) as e:
        D.dsa_sparse_mla_attn_noalloc(d, FAKE, FAKE, FAKE, 0.1, FAKE, stream=0)
    assert e.value.status == D.ERR_UNSUPPORTED and "at most" in str(e.value)
    # the 64-row decode step fits
    assert dsa.dsa_attn_workspace_size(_dims(batch=64, n_q=1, n_kv=131072, q_pos0=131071, topk=2048)) <= 40 << 20
    # the other checks are those of dsa_sparse_mla_attn
    with pytest.raises(dsa.DSAError) as e:
        D.dsa_sparse_mla_attn_noalloc(_dims(), FAKE, FAKE, FAKE, float("nan"), FAKE, stream=0)
    assert e.value.status == D.ERR_INVALID_ARG
