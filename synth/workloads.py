"""Named synthetic workloads and host-side input builders.

The five workloads mirror the shapes of the 128K-context DSA setting the
pages describe (k = 2048 selected tokens, 64 index heads of 128 dims, 128
attention heads over 576-d latents of which 512 are values):

  tiny   1 x 256, H_I=4 d_I=32, k=32, 8 heads, Dk=80 Dv=64 (all "fp32"
         draws, rounded to the kernel formats for the GPU path)
  p4k    1 x 4096 prefill
  p32k   1 x 32768 prefill; latents and index keys share a rank-32 factor
  p128k  1 x 131072 prefill
  dec64  64 sequences x 1 new token against a 131072-token cache

Flat element numbering of every tensor (row-major) is fixed here and in the
device filler, so host and device produce identical bytes:

  q_idx [B,T,H_I,d_I] token = b*T+i   (FP8, per-token scale over H_I*d_I)
  w_idx [B,T,H_I]                      (bf16, z * 2^w_exp2)
  k_idx [B,S,d_I]     token = b*S+s   (FP8, per-token scale over d_I)
  q     [B,T,H,Dk]                     (bf16)
  kv    [B,S,Dk]                       (bf16)
"""
from __future__ import annotations

import dataclasses
import math
from functools import lru_cache

import numpy as np

from . import gen


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q: int
    n_kv: int
    q_pos0: int
    idx_heads: int
    idx_dim: int
    heads: int
    dim_qk: int
    dim_v: int
    topk: int
    w_exp2: int          # w = z * 2^w_exp2
    sm_scale: float
    low_rank: bool
    seed: int

    # ---- derived sizes (Sec. 1.1 cost figures: 8192 MAC per indexer pair,
    # 128 * (576 + 512) MAC per selected pair)
    def positions(self):
        return np.arange(self.q_pos0, self.q_pos0 + self.n_q)

    def causal_pairs(self) -> int:
        p = self.positions()
        return int(self.batch * np.minimum(p + 1, self.n_kv).sum())

    def selected_pairs(self) -> int:
        p = self.positions()
        return int(self.batch * np.minimum(self.topk, np.minimum(p + 1, self.n_kv)).sum())

    def indexer_flop(self) -> float:
        return 2.0 * self.causal_pairs() * self.idx_heads * self.idx_dim

    def attn_flop(self) -> float:
        return 2.0 * self.selected_pairs() * self.heads * (self.dim_qk + self.dim_v)

    def dims_tuple(self):
        return (self.batch, self.n_q, self.n_kv, self.q_pos0, self.idx_heads, self.idx_dim,
                self.heads, self.dim_qk, self.dim_v, self.topk)


def _seed(i: int) -> int:
    return 0xD5A0 + i


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 256, 0, 4, 32, 8, 80, 64, 32, -1, 1.0 / math.sqrt(80), False, _seed(0)),
    "p4k": Workload("p4k", 1, 4096, 4096, 0, 64, 128, 128, 576, 512, 2048, -3, 1.0 / math.sqrt(192), False, _seed(1)),
    "p32k": Workload("p32k", 1, 32768, 32768, 0, 64, 128, 128, 576, 512, 2048, -3, 1.0 / math.sqrt(192), True, _seed(2)),
    "p128k": Workload("p128k", 1, 131072, 131072, 0, 64, 128, 128, 576, 512, 2048, -3, 1.0 / math.sqrt(192), False, _seed(3)),
    "dec64": Workload("dec64", 64, 1, 131072, 131071, 64, 128, 128, 576, 512, 2048, -3, 1.0 / math.sqrt(192), False, _seed(4)),
}

LOW_RANK = 32
LOW_RANK_NOISE = 0.3


def custom(base: str, **kw) -> Workload:
    """A variant of a named workload (edge cases: other T, S, k, q_pos0...)."""
    return dataclasses.replace(WORKLOADS[base], **kw)


# ----------------------------------------------------------------- raw draws
def raw_q_idx(wl: Workload, b: int, rows) -> np.ndarray:
    """float32 [n, H_I, d_I] before quantisation."""
    tl = wl.idx_heads * wl.idx_dim
    out = [gen.normal_f32(wl.seed, gen.TID["q_idx"], (b * wl.n_q + int(i)) * tl, tl) for i in rows]
    return np.stack(out).reshape(len(out), wl.idx_heads, wl.idx_dim) if out else np.zeros((0, wl.idx_heads, wl.idx_dim), np.float32)


def raw_w_idx(wl: Workload, b: int, rows) -> np.ndarray:
    h = wl.idx_heads
    mul = np.float32(2.0 ** wl.w_exp2)
    out = [gen.normal_f32(wl.seed, gen.TID["w_idx"], (b * wl.n_q + int(i)) * h, h) * mul for i in rows]
    return np.stack(out).astype(np.float32) if out else np.zeros((0, h), np.float32)


@lru_cache(maxsize=4)
def _low_rank(wl: Workload):
    assert wl.batch == 1
    return gen.low_rank_rows(wl.seed, wl.n_kv, LOW_RANK, wl.dim_qk, wl.idx_dim, LOW_RANK_NOISE)


def raw_k_idx(wl: Workload, b: int, s0: int, s1: int) -> np.ndarray:
    """float32 [s1-s0, d_I] keys of sequence b before quantisation."""
    if wl.low_rank:
        return _low_rank(wl)[1][s0:s1]
    d = wl.idx_dim
    return gen.normal_f32(wl.seed, gen.TID["k_idx"], (b * wl.n_kv + s0) * d, (s1 - s0) * d).reshape(s1 - s0, d)


def raw_q(wl: Workload, b: int, rows) -> np.ndarray:
    hd = wl.heads * wl.dim_qk
    out = [gen.normal_f32(wl.seed, gen.TID["q"], (b * wl.n_q + int(i)) * hd, hd) for i in rows]
    return np.stack(out).reshape(len(out), wl.heads, wl.dim_qk) if out else np.zeros((0, wl.heads, wl.dim_qk), np.float32)


def raw_kv_rows(wl: Workload, b: int, srows) -> np.ndarray:
    """float32 [n, Dk] latent rows (arbitrary row list) before bf16 rounding."""
    srows = np.asarray(srows, dtype=np.int64)
    if wl.low_rank:
        return _low_rank(wl)[0][srows]
    d = wl.dim_qk
    out = np.empty((len(srows), d), dtype=np.float32)
    # group consecutive runs for speed
    start = 0
    while start < len(srows):
        end = start + 1
        while end < len(srows) and srows[end] == srows[end - 1] + 1:
            end += 1
        s0 = int(srows[start])
        out[start:end] = gen.normal_f32(wl.seed, gen.TID["kv"], (b * wl.n_kv + s0) * d, (end - start) * d).reshape(end - start, d)
        start = end
    return out


# ----------------------------------------------------------------- kernel formats
def q_idx_fp8(wl: Workload, b: int, rows):
    """(codes uint8 [n, H_I, d_I], scales float32 [n])."""
    raw = raw_q_idx(wl, b, rows)
    codes, scales = gen.quantize_tokens_e4m3(raw.reshape(raw.shape[0], -1))
    return codes.reshape(raw.shape), scales


def k_idx_fp8(wl: Workload, b: int, s0: int, s1: int):
    codes, scales = gen.quantize_tokens_e4m3(raw_k_idx(wl, b, s0, s1))
    return codes, scales


def w_idx_bf16(wl: Workload, b: int, rows) -> np.ndarray:
    return gen.f32_to_bf16_bits(raw_w_idx(wl, b, rows))


def q_bf16(wl: Workload, b: int, rows) -> np.ndarray:
    return gen.f32_to_bf16_bits(raw_q(wl, b, rows))


def kv_bf16_rows(wl: Workload, b: int, srows) -> np.ndarray:
    return gen.f32_to_bf16_bits(raw_kv_rows(wl, b, srows))


def host_inputs(wl: Workload):
    """All inputs of a (small) workload in kernel formats, as numpy arrays."""
    B, T, S = wl.batch, wl.n_q, wl.n_kv
    rows = range(T)
    qc, qs, w, kc, ks, q, kv = [], [], [], [], [], [], []
    for b in range(B):
        c, s = q_idx_fp8(wl, b, rows); qc.append(c); qs.append(s)
        w.append(w_idx_bf16(wl, b, rows))
        c, s = k_idx_fp8(wl, b, 0, S); kc.append(c); ks.append(s)
        q.append(q_bf16(wl, b, rows))
        kv.append(kv_bf16_rows(wl, b, np.arange(S)))
    return {
        "q_idx": np.stack(qc), "q_scale": np.stack(qs), "w_idx": np.stack(w),
        "k_idx": np.stack(kc), "k_scale": np.stack(ks), "q": np.stack(q), "kv": np.stack(kv),
    }


# ----------------------------------------------------------------- MHA mode (masked short prefill)
def mha_dims(wl: Workload):
    """(dn, dr, dvh): per-head decompressed key dims, shared rope dims and
    value dims of MHA mode.  128 / 64 / 128 for 576-d latents with 512
    compressed dims (a 192-d per-head query, matching the 1/sqrt(192)
    softmax scale); half the compressed width for the small shapes."""
    dr = wl.dim_qk - wl.dim_v
    dn = 128 if wl.dim_v >= 512 else wl.dim_v // 2
    return dn, dr, dn


def mha_w_exp2(wl: Workload) -> int:
    """Decompression weights are z * 2^e with 2^e close to 1/sqrt(dim_v), so
    the per-head keys and values have about unit size."""
    return -int(math.floor(math.log2(wl.dim_v) / 2))


def q_mha_bf16(wl: Workload, b: int, rows) -> np.ndarray:
    """bf16 bits [n, H, dn + dr] of the MHA-mode queries of rows `rows`."""
    dn, dr, _ = mha_dims(wl)
    hd = wl.heads * (dn + dr)
    out = [gen.normal_f32(wl.seed, gen.TID["q_mha"], (b * wl.n_q + int(i)) * hd, hd) for i in rows]
    raw = np.stack(out) if out else np.zeros((0, hd), np.float32)
    return gen.f32_to_bf16_bits(raw).reshape(len(out), wl.heads, dn + dr)


def w_mha_bf16(wl: Workload, which: str) -> np.ndarray:
    """bf16 bits of W_UK [H, dn, dim_v] ("w_uk") or W_UV [H, dvh, dim_v] ("w_uv")."""
    dn, _, dvh = mha_dims(wl)
    rows = dn if which == "w_uk" else dvh
    n = wl.heads * rows * wl.dim_v
    raw = gen.normal_f32(wl.seed, gen.TID[which], 0, n) * np.float32(2.0 ** mha_w_exp2(wl))
    return gen.f32_to_bf16_bits(raw.astype(np.float32)).reshape(wl.heads, rows, wl.dim_v)


# ----------------------------------------------------------------- paged / variable-length layouts
@dataclasses.dataclass(frozen=True)
class PagedLayout:
    """Per-sequence lengths and a page placement for workload `base`:
    sequence b holds seq_lens[b] tokens; its logical page j lives in
    physical page table[b, j] of a pool of num_pages pages."""
    page_size: int
    seq_lens: tuple
    table: np.ndarray      # int32 [B, max_pages]
    num_pages: int

    @property
    def max_pages(self) -> int:
        return int(self.table.shape[1])


def paged_layout(wl: Workload, page_size: int, min_len: int | None = None, spare_pages: int = 3,
                 full: bool = False) -> PagedLayout:
    """Seeded layout: lengths uniform in [min_len, n_kv] (all n_kv if `full`),
    at least n_q; every sequence owns ceil(n_kv / page_size) pages, placed at
    random in a pool that also holds `spare_pages` unused pages."""
    rs = np.random.RandomState(wl.seed + 7919)
    lo = max(wl.n_q, min_len if min_len is not None else wl.n_q)
    if full:
        lens = [wl.n_kv] * wl.batch
    else:
        lens = [int(x) for x in rs.randint(lo, wl.n_kv + 1, size=wl.batch)]
    max_pages = (wl.n_kv + page_size - 1) // page_size
    num_pages = wl.batch * max_pages + spare_pages
    table = rs.permutation(num_pages)[:wl.batch * max_pages].reshape(wl.batch, max_pages).astype(np.int32)
    return PagedLayout(page_size, tuple(lens), table, num_pages)


def pool_rows(layout: PagedLayout, b: int, s) -> np.ndarray:
    """Pool rows of tokens s (array) of sequence b."""
    s = np.asarray(s, dtype=np.int64)
    return layout.table[b, s // layout.page_size].astype(np.int64) * layout.page_size + s % layout.page_size
