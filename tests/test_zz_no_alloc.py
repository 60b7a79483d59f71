"""dsa_sparse_mla_attn_noalloc (split partials in the library's static device
array, no workspace) against dsa_sparse_mla_attn with a caller workspace, on
two calls in a row, the second with a smaller input: the outputs agree bit
for bit, and both meet the oracle tolerance on sampled rows."""
import numpy as np
import pytest
import torch

import sparse_attention_long_amd as dsa
from synth import device as SD
from synth import workloads as W

from dsa_parity import ATTN_MAX_REL, LSE_ABS, HostSide, attn_errors, bf16_tensor_to_f64, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()
    yield
    torch.cuda.synchronize()


def _selection(wl, rs):
    """Sorted random selections; sequence 1 is short (padding), sequence 2 empty."""
    B, k, S = wl.batch, wl.topk, wl.n_kv
    idx = np.full((B, 1, k), -1, np.int32)
    for b in range(B):
        m = k if b not in (1, 2) else (700 if b == 1 else 0)
        idx[b, 0, :m] = np.sort(rs.choice(S, size=m, replace=False))
    return idx


def _run_both(wl, seed):
    d = SD.fill_inputs(wl)
    dims = dsa.Dims.of(wl)
    idx = to_dev(_selection(wl, np.random.RandomState(seed)))
    shape_o = (wl.batch, 1, wl.heads, wl.dim_v)
    out_ws = torch.full(shape_o, 7, dtype=torch.int16, device="cuda")
    lse_ws = torch.full((wl.batch, 1, wl.heads), 7.0, dtype=torch.float32, device="cuda")
    nws = dsa.dsa_attn_workspace_size(dims)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    dsa.dsa_sparse_mla_attn(dims, d["q"], d["kv"], idx, wl.sm_scale, out_ws, lse_ws, ws, nws)
    out_na = torch.full(shape_o, -7, dtype=torch.int16, device="cuda")
    lse_na = torch.full((wl.batch, 1, wl.heads), -7.0, dtype=torch.float32, device="cuda")
    dsa.dsa.dsa_sparse_mla_attn_noalloc(dims, d["q"], d["kv"], idx, wl.sm_scale, out_na, lse_na)
    torch.cuda.synchronize()
    return nws, idx.cpu().numpy(), (out_ws, lse_ws), (out_na, lse_na)


def _check_oracle(wl, idx, out, lse, rows):
    worst, worst_lse = 0.0, 0.0
    for b in rows:
        sel = idx[b, 0]
        o = bf16_tensor_to_f64(out[b, 0])
        l = lse[b, 0].cpu().numpy()
        if not np.any(sel >= 0):
            assert np.all(o == 0) and np.all(np.isneginf(l))
            continue
        ref_o, ref_lse = HostSide(wl, b).attention(0, sel)
        worst = max(worst, attn_errors(o, ref_o).max())
        worst_lse = max(worst_lse, np.abs(l - ref_lse).max())
    return worst, worst_lse


def test_noalloc_matches_workspace_call_on_two_calls():
    # first call: 64 decode rows (4 splits per row, 33.7 MB of partials);
    # second call: 8 rows (16 splits per row, 16.8 MB), which leaves the
    # first call's partials in the array's upper part untouched
    for B, S, seed in ((64, 9000, 21), (8, 5000, 22)):
        wl = W.custom("dec64", batch=B, n_kv=S, q_pos0=S - 1)
        nws, idx, (o_ws, l_ws), (o_na, l_na) = _run_both(wl, seed)
        print(f"B={B}: partials {nws} bytes", flush=True)
        assert nws > 0
        assert torch.equal(o_ws, o_na), B
        assert torch.equal(l_ws.view(torch.int32), l_na.view(torch.int32)), B
        worst, wlse = _check_oracle(wl, idx, o_na, l_na, (0, 1, 2, B - 1))
        print(f"B={B}: max rel err {worst:.3e}, lse {wlse:.3e}", flush=True)
        assert worst <= ATTN_MAX_REL and wlse <= LSE_ABS
