"""Device-side filling of workload inputs (HIP generator library via ctypes,
torch for device memory).  Produces the same bytes as the host builders in
``workloads.py``."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import gen
from .workloads import Workload, _low_rank
from .workloads import pool_rows as W_pool_rows

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa_synth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_fill_bf16.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.synth_fill_f32.argtypes = L.synth_fill_bf16.argtypes
        L.synth_fill_e4m3_tokens.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.synth_stream_key.argtypes = [ctypes.c_uint64, ctypes.c_int32]
        L.synth_stream_key.restype = ctypes.c_uint64
        _lib = L
    return _lib


def _check(rc):
    if rc != 0:
        raise RuntimeError(f"synth device fill failed: hipError {rc}")


def _stream(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def fill_inputs(wl: Workload, device="cuda"):
    """Allocate and fill all inputs of `wl` on the device.  Returns a dict of
    torch tensors: q_idx uint8 [B,T,HI,dI], q_scale f32 [B,T], w_idx int16
    (bf16 bits) [B,T,HI], k_idx uint8 [B,S,dI], k_scale f32 [B,S],
    q int16 [B,T,H,Dk], kv int16 [B,S,Dk]."""
    import torch
    L = lib()
    B, T, S = wl.batch, wl.n_q, wl.n_kv
    HI, dI, H, Dk = wl.idx_heads, wl.idx_dim, wl.heads, wl.dim_qk
    st = _stream(torch)
    t = {
        "q_idx": torch.empty((B, T, HI, dI), dtype=torch.uint8, device=device),
        "q_scale": torch.empty((B, T), dtype=torch.float32, device=device),
        "w_idx": torch.empty((B, T, HI), dtype=torch.int16, device=device),
        "k_idx": torch.empty((B, S, dI), dtype=torch.uint8, device=device),
        "k_scale": torch.empty((B, S), dtype=torch.float32, device=device),
        "q": torch.empty((B, T, H, Dk), dtype=torch.int16, device=device),
        "kv": torch.empty((B, S, Dk), dtype=torch.int16, device=device),
    }
    _check(L.synth_fill_e4m3_tokens(wl.seed, gen.TID["q_idx"], 0, B * T, HI * dI,
                                    t["q_idx"].data_ptr(), t["q_scale"].data_ptr(), st))
    _check(L.synth_fill_bf16(wl.seed, gen.TID["w_idx"], 0, B * T * HI, wl.w_exp2, t["w_idx"].data_ptr(), st))
    _check(L.synth_fill_bf16(wl.seed, gen.TID["q"], 0, B * T * H * Dk, 0, t["q"].data_ptr(), st))
    if wl.low_rank:
        c, k = _low_rank(wl)
        codes, scales = gen.quantize_tokens_e4m3(k)
        t["k_idx"].copy_(torch.from_numpy(codes).reshape(B, S, dI))
        t["k_scale"].copy_(torch.from_numpy(scales).reshape(B, S))
        t["kv"].copy_(torch.from_numpy(gen.f32_to_bf16_bits(c).view(np.int16)).reshape(B, S, Dk))
    else:
        _check(L.synth_fill_e4m3_tokens(wl.seed, gen.TID["k_idx"], 0, B * S, dI,
                                        t["k_idx"].data_ptr(), t["k_scale"].data_ptr(), st))
        _check(L.synth_fill_bf16(wl.seed, gen.TID["kv"], 0, B * S * Dk, 0, t["kv"].data_ptr(), st))
    return t


def fill_mha(wl: Workload, device="cuda"):
    """MHA-mode inputs of `wl` on the device: q_mha int16 (bf16 bits)
    [B,T,H,dn+dr], w_uk [H,dn,Dv], w_uv [H,dvh,Dv]."""
    import torch
    from .workloads import mha_dims, mha_w_exp2
    L = lib()
    B, T, H, Dv = wl.batch, wl.n_q, wl.heads, wl.dim_v
    dn, dr, dvh = mha_dims(wl)
    st = _stream(torch)
    t = {
        "q_mha": torch.empty((B, T, H, dn + dr), dtype=torch.int16, device=device),
        "w_uk": torch.empty((H, dn, Dv), dtype=torch.int16, device=device),
        "w_uv": torch.empty((H, dvh, Dv), dtype=torch.int16, device=device),
    }
    _check(L.synth_fill_bf16(wl.seed, gen.TID["q_mha"], 0, t["q_mha"].numel(), 0, t["q_mha"].data_ptr(), st))
    e = mha_w_exp2(wl)
    _check(L.synth_fill_bf16(wl.seed, gen.TID["w_uk"], 0, t["w_uk"].numel(), e, t["w_uk"].data_ptr(), st))
    _check(L.synth_fill_bf16(wl.seed, gen.TID["w_uv"], 0, t["w_uv"].numel(), e, t["w_uv"].data_ptr(), st))
    return t


def fill_paged(wl: Workload, layout, device="cuda"):
    """Inputs of `wl` with the caches moved into page pools per `layout`
    (synth.workloads.PagedLayout): the dict of fill_inputs with k_idx,
    k_scale and kv replaced by pools [num_pages * page_size, ...] (slots of
    unused pages and past a sequence's capacity hold zeros), plus the device
    int32 tensors seq_lens [B] and page_table [B, max_pages]."""
    import torch
    t = fill_inputs(wl, device)
    B, S, P = wl.batch, wl.n_kv, layout.page_size
    rows = layout.num_pages * P
    slots = torch.from_numpy(np.stack([W_pool_rows(layout, b, np.arange(S)) for b in range(B)])).to(device)
    for name, tail in (("k_idx", (wl.idx_dim,)), ("k_scale", ()), ("kv", (wl.dim_qk,))):
        dense = t[name]
        pool = torch.zeros((rows,) + tail, dtype=dense.dtype, device=device)
        pool.index_copy_(0, slots.reshape(-1), dense.reshape((B * S,) + tail))
        t[name] = pool
        del dense
    t["seq_lens"] = torch.tensor(layout.seq_lens, dtype=torch.int32, device=device)
    t["page_table"] = torch.from_numpy(layout.table).to(device)
    return t
