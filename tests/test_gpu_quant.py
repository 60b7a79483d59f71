"""GPU parity of the per-token FP8 quantisation and of the decode cache
append (through the C ABI) against the oracle.  Codes and scales are byte
work: the comparison is bit-exact."""
import numpy as np
import pytest
import torch

import sparse_attention_long_amd as dsa
from oracle import dsa_oracle as O
from sparse_attention_long_amd.dsa import Dims
from synth import gen
from synth import workloads as W

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


def quant_gpu(x: np.ndarray, bf16: bool = False):
    n, L = x.shape
    if bf16:
        xd = torch.from_numpy(gen.f32_to_bf16_bits(x).view(np.int16)).cuda()
    else:
        xd = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    codes = torch.full((n, L), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa.dsa_quantize_e4m3(xd, n, L, codes, scales, dtype=1 if bf16 else 0)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _tie_row():
    vals = O.E4M3_VALUES[:0x7F]
    row = np.concatenate([[448.0], vals, -vals, (vals[:-1] + vals[1:]) / 2, -(vals[:-1] + vals[1:]) / 2])
    return np.concatenate([row, np.zeros((-len(row)) % 4)]).astype(np.float32)[None, :]


def _cases():
    rs = np.random.RandomState(21)
    c = {
        "spread_128": (rs.randn(257, 128) * np.exp(rs.randn(257, 1) * 4)).astype(np.float32),
        "query_8192": rs.randn(5, 8192).astype(np.float32),
        "len_4": rs.randn(33, 4).astype(np.float32),
        "len_1024": rs.standard_cauchy((9, 1024)).astype(np.float32),
        "len_1028": rs.standard_cauchy((9, 1028)).astype(np.float32),
        "tiny_and_huge": np.concatenate([rs.randn(4, 64) * 1e-30, rs.randn(4, 64) * 1e30]).astype(np.float32),
        "ties": _tie_row(),
    }
    z = rs.randn(6, 128).astype(np.float32)
    z[0] = 0.0
    z[1] = -0.0
    z[2, :] = 0.0
    z[2, 17] = -5.0
    c["zeros"] = z
    return c


CASES = _cases()


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_matches_oracle(name, bf16):
    x = CASES[name]
    if bf16:   # the oracle sees the bf16-rounded values the kernel reads
        x = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(x))
    codes, scales = quant_gpu(x, bf16=bf16)
    rc, rsc = O.quantize_e4m3_tokens(x)
    assert np.array_equal(scales.view(np.uint32), rsc.view(np.uint32)), name
    bad = np.argwhere(codes != rc)
    assert bad.size == 0, (name, bad[:5], codes[tuple(bad[0])], rc[tuple(bad[0])])


def test_quantize_reproduces_the_workload_inputs():
    # The FP8 inputs every other test feeds the indexer come from the host
    # quantiser of the input generator; the GPU call must give the same bytes.
    wl = W.WORKLOADS["p4k"]
    rows = [0, 1, 777, 4095]
    raw = W.raw_q_idx(wl, 0, rows).reshape(len(rows), -1)
    codes, scales = quant_gpu(raw)
    c, s = W.q_idx_fp8(wl, 0, rows)
    assert np.array_equal(codes, c.reshape(len(rows), -1)) and np.array_equal(scales, s)
    rawk = W.raw_k_idx(wl, 0, 100, 612)
    codes, scales = quant_gpu(rawk)
    c, s = W.k_idx_fp8(wl, 0, 100, 612)
    assert np.array_equal(codes, c) and np.array_equal(scales, s)


@pytest.mark.parametrize("bf16", [False, True])
def test_cache_append_matches_oracle(bf16):
    rs = np.random.RandomState(22)
    B, S, T, pos0, dI, Dk = 3, 50, 2, 37, 128, 576
    kc = rs.randint(0, 256, size=(B, S, dI)).astype(np.uint8)
    ks = rs.rand(B, S).astype(np.float32)
    kv = rs.randint(0, 1 << 15, size=(B, S, Dk)).astype(np.uint16)
    k_new = rs.randn(B, T, dI).astype(np.float32)
    if bf16:
        k_new = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(k_new))
    kv_new = rs.randint(0, 1 << 15, size=(B, T, Dk)).astype(np.uint16)
    dk = torch.from_numpy(kc).cuda()
    dks = torch.from_numpy(ks).cuda()
    dkv = torch.from_numpy(kv.view(np.int16)).cuda()
    kn = torch.from_numpy(gen.f32_to_bf16_bits(k_new).view(np.int16) if bf16 else k_new).cuda()
    dims = Dims(batch=B, n_q=T, n_kv=S, q_pos0=pos0, idx_heads=64, idx_dim=dI, heads=128, dim_qk=Dk, dim_v=512,
                topk=16)
    dsa.dsa.dsa_cache_append(dims, kn, dk, dks, kv_new=torch.from_numpy(kv_new.view(np.int16)).cuda(), kv=dkv,
                             k_dtype=1 if bf16 else 0)
    torch.cuda.synchronize()
    rk, rks, rkv = O.cache_append(kc, ks, kv, k_new, kv_new, pos0)
    assert np.array_equal(dk.cpu().numpy(), rk)
    assert np.array_equal(dks.cpu().numpy().view(np.uint32), rks.view(np.uint32))
    assert np.array_equal(dkv.cpu().numpy().view(np.uint16), rkv)
    _say("cache append ok", "bf16" if bf16 else "f32")


def test_cache_append_keys_only():
    rs = np.random.RandomState(23)
    B, S, T, pos0, dI = 2, 9, 1, 8, 32
    kc = np.zeros((B, S, dI), np.uint8)
    ks = np.ones((B, S), np.float32)
    k_new = rs.randn(B, T, dI).astype(np.float32)
    dk, dks = torch.from_numpy(kc).cuda(), torch.from_numpy(ks).cuda()
    dims = Dims(batch=B, n_q=T, n_kv=S, q_pos0=pos0, idx_heads=4, idx_dim=dI, heads=8, dim_qk=80, dim_v=64, topk=4)
    dsa.dsa.dsa_cache_append(dims, torch.from_numpy(k_new).cuda(), dk, dks, k_dtype=0)
    torch.cuda.synchronize()
    rk, rks, _ = O.cache_append(kc, ks, None, k_new, None, pos0)
    assert np.array_equal(dk.cpu().numpy(), rk) and np.array_equal(dks.cpu().numpy(), rks)
