"""Seeded synthetic inputs: determinism, distribution, and exact agreement of
the storage-format rounding with torch's conversions."""
import numpy as np
import torch

from synth import gen, workloads as W


def test_counter_based_slices_are_consistent():
    a = gen.normal_f32(7, 3, 0, 1000)
    b = gen.normal_f32(7, 3, 400, 200)
    assert np.array_equal(a[400:600], b)
    assert not np.array_equal(gen.normal_f32(7, 4, 0, 1000), a)      # other tensor id
    assert not np.array_equal(gen.normal_f32(8, 3, 0, 1000), a)      # other seed


def test_irwin_hall_moments_and_support():
    z = gen.normal_f32(1, 1, 0, 2_000_000).astype(np.float64)
    assert abs(z.mean()) < 3e-3 and abs(z.var() - 1) < 5e-3
    assert z.min() >= -6 and z.max() <= 6
    # values are exact multiples of 2^-20 (the sum is formed in integers)
    assert np.all(z * 2 ** 20 == np.round(z * 2 ** 20))


def test_bf16_rounding_matches_torch():
    x = gen.normal_f32(2, 1, 0, 100000) * np.float32(37.0)
    mine = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(gen.bf16_bits_to_f32(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_e4m3_rounding_matches_torch_below_saturation():
    rs = np.random.RandomState(0)
    x = np.concatenate([rs.randn(50000) * 60, rs.randn(20000) * 1e-2, rs.uniform(-463.9, 463.9, 20000),
                        np.ldexp(np.arange(1, 64), -9), 2.0 ** np.arange(-9, 9)]).astype(np.float32)
    mine = gen.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_saturates_instead_of_nan():
    x = np.array([464.0, 479.0, 500.0, 1e6, -1e6], dtype=np.float32)
    assert list(gen.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_per_token_quantisation():
    x = gen.normal_f32(3, 1, 0, 64 * 128).reshape(64, 128)
    x[5] = 0.0
    codes, scales = gen.quantize_tokens_e4m3(x)
    amax = np.abs(x).max(axis=1)
    assert scales[5] == 1.0 and np.all(codes[5] == 0)
    nz = np.arange(64) != 5
    assert np.array_equal(scales[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy() * scales[:, None]
    # relative error of E4M3 round-to-nearest is at most 2^-4 of the value (normal range)
    big = np.abs(x) > scales[:, None] * 2 ** -6
    assert np.all(np.abs(dec - x)[big] <= np.abs(x)[big] * 2 ** -4 * 1.0001)
    assert np.all(np.abs(dec).max(axis=1)[nz] <= 448 * scales[nz] * (1 + 1e-6))


def test_workload_shapes_and_counts():
    tiny = W.WORKLOADS["tiny"]
    assert tiny.causal_pairs() == 256 * 257 // 2 == 32896
    assert tiny.selected_pairs() == 7696
    p128 = W.WORKLOADS["p128k"]
    assert p128.causal_pairs() == 8_590_000_128
    assert p128.selected_pairs() == 266_339_328
    d = W.WORKLOADS["dec64"]
    assert d.causal_pairs() == 64 * 131072 and d.selected_pairs() == 64 * 2048


def test_host_inputs_tiny_formats():
    tiny = W.WORKLOADS["tiny"]
    h = W.host_inputs(tiny)
    assert h["q_idx"].shape == (1, 256, 4, 32) and h["q_idx"].dtype == np.uint8
    assert h["k_idx"].shape == (1, 256, 32) and h["k_scale"].shape == (1, 256)
    assert h["w_idx"].shape == (1, 256, 4) and h["q"].shape == (1, 256, 8, 80) and h["kv"].shape == (1, 256, 80)
    # row helpers regenerate the same bytes as the full tensors
    c, s = W.q_idx_fp8(tiny, 0, [17, 200])
    assert np.array_equal(c, h["q_idx"][0, [17, 200]]) and np.array_equal(s, h["q_scale"][0, [17, 200]])
    assert np.array_equal(W.kv_bf16_rows(tiny, 0, [3, 4, 9]), h["kv"][0, [3, 4, 9]])


def test_low_rank_rows_have_structure():
    c, k = gen.low_rank_rows(11, 512, 32, 64, 16)
    # the rank-32 part dominates: 32 singular values carry most of the energy
    sv = np.linalg.svd(c.astype(np.float64), compute_uv=False)
    assert (sv[:32] ** 2).sum() / (sv ** 2).sum() > 0.85
    assert c.shape == (512, 64) and k.shape == (512, 16)
