"""Benchmark of the DSA forward path on one MI355X.

One step = one dsa_forward over the whole workload (indexer -> top-k ->
sparse MLA for every query row), inputs already resident in HBM.  Prints one
JSON line:
  value        query-tokens/s of dsa_forward on the 128K prefill workload
  roofline     the dominant kernel's algorithmic throughput against its peak
  cpu_baseline the CPU oracle on a stratified row sample of the same workload
plus per-stage times, indexer FP8 TFLOP/s, the 32K prefill, the 64 x 128K
decode step and the other legs (paged decode, quantisation, short prefill).

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload p128k]
                       [--cpu-rows R] [--cpu-decode-seqs N] [--no-cpu-baseline] [--no-decode]
                       [--stage-reps N] [--short-prefill-only] [--calib-copy-mb M]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_FP8_TFLOPS = 5000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
METRIC = "DSA fwd query-tokens/sec at L=128K,k=2048; indexer FP8 TFLOP/s; decode GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """HIP events recorded on the stream the kernels are launched on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def start(self):
        """The opening event of a timed region, recorded behind torch's spin
        kernel (10^6 clock cycles, a fraction of a millisecond; it touches no
        memory, so it leaves no dirty lines in the caches), so that the host
        has enqueued the first timed calls before the GPU reaches the event:
        on an idle stream the region would also hold the host's enqueue
        latency of the first call."""
        with self.torch.cuda.stream(self.stream):
            self.torch.cuda._sleep(1_000_000)
        return self.event()


def alloc_forward(torch, wl, dsa):
    dims = dsa.Dims.of(wl)
    out = torch.empty((wl.batch, wl.n_q, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.batch, wl.n_q, wl.heads), dtype=torch.float32, device="cuda")
    nws = dsa.dsa_forward_workspace_size(dims)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    return dims, out, lse, ws, nws


def time_forward(torch, wl, d, dsa, steps, warmup, stream):
    dims, out, lse, ws, nws = alloc_forward(torch, wl, dsa)

    def step():
        dsa.dsa_forward(dims, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], d["q"], d["kv"],
                        wl.sm_scale, out, lse, None, ws, nws, stream=stream.cuda_stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = Timer(torch, stream)
    e0 = t.start()
    for _ in range(steps):
        step()
    e1 = t.event()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_forward_kl(torch, wl, d, dsa, steps, warmup, stream):
    """The sparse-stage training forward (dsa_forward_kl: the forward plus the
    indexer KL of Eq. (4) per row), whole-workload ms per step."""
    dims, out, lse, ws, nws = alloc_forward(torch, wl, dsa)
    kl = torch.empty((wl.batch, wl.n_q), dtype=torch.float32, device="cuda")

    def step():
        dsa.dsa.dsa_forward_kl(dims, None, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], d["q"],
                               d["kv"], wl.sm_scale, out, lse, None, kl, ws, nws, stream=stream.cuda_stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = Timer(torch, stream)
    e0 = t.start()
    for _ in range(steps):
        step()
    e1 = t.event()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, float(kl.double().mean().item())


def time_stages(torch, wl, d, dsa, reps, stream):
    """The forward's chunk loop through the three separate calls, with events
    between stages: the chunk rows and the top-k split come from the
    library's own plan (dsa_forward_plan_of), so every launch is the one
    dsa_forward makes.  Returns per-stage times, launches per stage and the
    forward's workspace size."""
    S, k = wl.n_kv, wl.topk
    full = dsa.Dims.of(wl)
    plan = dsa.dsa.dsa_forward_plan_of(full)
    tc = int(plan.chunk_rows)
    sc = torch.empty((wl.batch, tc, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((wl.batch, tc, k), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.batch, wl.n_q, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    lse = torch.empty((wl.batch, wl.n_q, wl.heads), dtype=torch.float32, device="cuda")
    assert wl.batch == 1 or tc == wl.n_q
    anws = dsa.dsa_attn_workspace_size(dsa.Dims.of(wl, n_q=tc))
    aws = torch.empty(max(anws, 1), dtype=torch.uint8, device="cuda")
    tnws = dsa.dsa.dsa_topk_workspace_size(dsa.Dims.of(wl, n_q=tc))
    tws = torch.empty(max(tnws, 1), dtype=torch.uint8, device="cuda")
    t = Timer(torch, stream)
    tot = {"indexer": 0.0, "topk": 0.0, "attention": 0.0}
    launches = 0
    s = stream.cuda_stream
    # The events are read once at the end, so the host enqueues ahead of the
    # GPU and each interval holds only the GPU's own work.
    torch.cuda.synchronize()
    marks = []
    first = True
    for _ in range(reps):
        for i0 in range(0, wl.n_q, tc):
            rows = min(tc, wl.n_q - i0)
            cd = dsa.Dims.of(wl, n_q=rows, q_pos0=wl.q_pos0 + i0)
            if wl.batch == 1:
                qi, qs, w = d["q_idx"][:, i0:], d["q_scale"][:, i0:], d["w_idx"][:, i0:]
                q, o, l = d["q"][:, i0:], out[:, i0:], lse[:, i0:]
            else:
                qi, qs, w, q, o, l = d["q_idx"], d["q_scale"], d["w_idx"], d["q"], out, lse
            e0 = t.start() if first else t.event()
            first = False
            dsa.dsa_indexer_scores(cd, qi, qs, w, d["k_idx"], d["k_scale"], sc, S, stream=s)
            e1 = t.event()
            dsa.dsa.dsa_topk_ws(cd, sc, S, idx, tws, tnws, stream=s)
            e2 = t.event()
            dsa.dsa_sparse_mla_attn(cd, q, d["kv"], idx, wl.sm_scale, o, l, aws, anws, stream=s)
            e3 = t.event()
            marks.append((e0, e1, e2, e3))
            launches += 1
    torch.cuda.synchronize()
    for e0, e1, e2, e3 in marks:
        tot["indexer"] += e0.elapsed_time(e1)
        tot["topk"] += e1.elapsed_time(e2)
        tot["attention"] += e2.elapsed_time(e3)
    return {k2: v / reps for k2, v in tot.items()}, launches // reps, int(plan.workspace_bytes)


# Dominant-kernel names per stage, the rocprofv3 summary that holds its
# measured HBM traffic, and the sources that summary was taken from.
STAGE_KERNELS = {
    "indexer": ("indexer_prefill_lds_kernel<4,4>", "indexer_prefill_lds_kernel_p128k.md", "indexer.hip"),
    "attention": ("sparse_mla_kernel<576,512,4>", "sparse_mla_kernel_p128k.md", "sparse_mla.hip"),
    "topk": ("topk_kernel", "topk_kernel_p128k.md", "topk.hip"),
}


def source_sha16(src):
    import hashlib
    h = hashlib.sha256()
    for f in (src, "dsa_device.h", "dsa_internal.h"):
        with open(os.path.join(ROOT, "sparse_attention_long_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(stage, workload):
    """HBM bytes per launch of the stage's kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None if there is none for this workload
    or the kernel's sources changed since it was taken."""
    if workload != "p128k":
        return None
    _, md, src = STAGE_KERNELS[stage]
    path = os.path.join(ROOT, "profiles", md)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256_16"):
                k, v = line.split(":", 1)
                vals[k] = v.split()[0]
    if vals.get("source_sha256_16") != source_sha16(src) or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def time_quantize(torch, dsa, wl, stream, reps=5):
    """Per-token FP8 quantisation of the workload's index keys (f32, [S, d_I])
    and of 16384 query tokens (bf16, [16384, H_I * d_I]): HBM-bound, reported
    as algorithmic GB/s (values read + codes and scales written)."""
    from synth import gen
    from synth.device import lib as synth_lib, _check
    L = synth_lib()
    S, dI, tq = wl.n_kv, wl.idx_dim, 16384
    ql = wl.idx_heads * wl.idx_dim
    kx = torch.empty((S, dI), dtype=torch.float32, device="cuda")
    qx = torch.empty((tq, ql), dtype=torch.int16, device="cuda")
    _check(L.synth_fill_f32(wl.seed, gen.TID["k_idx"], 0, S * dI, 0, kx.data_ptr(), stream.cuda_stream))
    _check(L.synth_fill_bf16(wl.seed, gen.TID["q_idx"], 0, tq * ql, 0, qx.data_ptr(), stream.cuda_stream))
    kc = torch.empty((S, dI), dtype=torch.uint8, device="cuda")
    ks = torch.empty((S,), dtype=torch.float32, device="cuda")
    qc = torch.empty((tq, ql), dtype=torch.uint8, device="cuda")
    qs = torch.empty((tq,), dtype=torch.float32, device="cuda")
    res = {}
    for name, x, n, ln, c, sc, dt, eb in (("index_keys_f32", kx, S, dI, kc, ks, 0, 4), ("queries_bf16", qx, tq, ql, qc, qs, 1, 2)):
        dsa.dsa.dsa_quantize_e4m3(x, n, ln, c, sc, dtype=dt, stream=stream.cuda_stream)
        torch.cuda.synchronize()
        t = Timer(torch, stream)
        e0 = t.start()
        for _ in range(reps):
            dsa.dsa.dsa_quantize_e4m3(x, n, ln, c, sc, dtype=dt, stream=stream.cuda_stream)
        e1 = t.event()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = n * ln * (eb + 1) + 4 * n
        res[name] = {"tokens": n, "token_len": ln, "us": ms * 1e3, "GB_per_s": nbytes / (ms / 1e3) / 1e9,
                     "frac_of_hbm_peak": nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}
    del kx, qx, kc, ks, qc, qs
    return res


def time_decode_paged(torch, dsa, stream, reps=10, warmup=2):
    """The decode step over paged, variable-length caches: 64 sequences with
    lengths uniform in [64K, 128K] tokens, 64-token pages placed at random in
    one pool.  Times dsa_forward_paged and the three paged calls separately,
    and reports the selections' locality counters (dsa_gather_stats)."""
    from synth import workloads as W
    from synth.device import fill_paged
    D = dsa.dsa
    wl = W.WORKLOADS["dec64"]
    P = 64
    lay = W.paged_layout(wl, P, min_len=wl.n_kv // 2)
    d = fill_paged(wl, lay)
    pk = D.PagedKV.of(d["seq_lens"], d["page_table"], P, lay.max_pages, lay.num_pages)
    dims = D.Dims.of(wl)
    B, S, k = wl.batch, wl.n_kv, wl.topk
    out = torch.empty((B, 1, wl.heads, wl.dim_v), dtype=torch.int16, device="cuda")
    idx = torch.empty((B, 1, k), dtype=torch.int32, device="cuda")
    fws = D.dsa_forward_workspace_size(dims)
    ws = torch.empty(fws, dtype=torch.uint8, device="cuda")
    sc = torch.empty((B, 1, S), dtype=torch.float32, device="cuda")
    nws = D.dsa_attn_workspace_size(dims)
    aws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    stats = torch.empty((B, 1, 3), dtype=torch.int32, device="cuda")
    st = stream.cuda_stream
    args = (d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"])

    def fwd():
        D.dsa_forward_paged(dims, pk, *args, d["q"], d["kv"], wl.sm_scale, out, None, idx, ws, fws, stream=st)

    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()
    t = Timer(torch, stream)
    e0 = t.start()
    for _ in range(reps):
        fwd()
    e1 = t.event()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / reps
    tot = {"indexer": 0.0, "topk": 0.0, "attention": 0.0, "gather_stats": 0.0}
    for _ in range(reps):
        ev = [t.start()]
        D.dsa_indexer_scores_paged(dims, pk, *args, sc, S, stream=st)
        ev.append(t.event())
        D.dsa_topk_paged(dims, pk, sc, S, idx, stream=st)
        ev.append(t.event())
        D.dsa_sparse_mla_attn_paged(dims, pk, d["q"], d["kv"], idx, wl.sm_scale, out, None, aws, nws, stream=st)
        ev.append(t.event())
        D.dsa_gather_stats(dims, P, idx, stats, stream=st)
        ev.append(t.event())
        torch.cuda.synchronize()
        for j, name in enumerate(tot):
            tot[name] += ev[j].elapsed_time(ev[j + 1]) / reps
    lens = np.array(lay.seq_lens, dtype=np.int64)
    sel = np.minimum(k, lens)
    idx_bytes = int((lens * (wl.idx_dim + 4)).sum() + B * wl.idx_heads * (wl.idx_dim + 2) + 4 * B
                    + 4 * lens.sum())
    topk_b = int(4 * lens.sum() + 4 * B * k)
    mla_bytes = int((sel * wl.dim_qk * 2).sum() + B * wl.heads * wl.dim_qk * 2 + B * wl.heads * wl.dim_v * 2)
    step_bytes = idx_bytes + topk_b + mla_bytes
    st_np = stats.cpu().numpy().reshape(B, 3).astype(np.float64)
    res = {"workload": "dec64 paged: 64 x [64K, 128K] tokens, 64-token pages", "page_size": P,
           "mean_seq_len": float(lens.mean()), "ms_per_step": step_ms,
           "GB_per_s": step_bytes / (step_ms / 1e3) / 1e9, "stages_ms": tot,
           "indexer_GB_per_s": idx_bytes / (tot["indexer"] / 1e3) / 1e9,
           "mla_gather_GB_per_s": mla_bytes / (tot["attention"] / 1e3) / 1e9,
           "algorithmic_bytes_per_step": step_bytes,
           "selection_locality": {"mean_pages": float(st_np[:, 0].mean()), "mean_runs": float(st_np[:, 1].mean()),
                                  "mean_max_hits_per_page": float(st_np[:, 2].mean())}}
    del d
    return res


def time_short_prefill(torch, dsa, stream, reps=5, warmup=2):
    """Short prefill (p4k: 4096 tokens, k = 2048) two ways: the sparse MQA-mode
    forward (dsa_forward) and the masked MHA mode that simulates it
    (dsa_masked_mha_forward), plus the masked path's stages through the
    separate calls."""
    from synth import workloads as W
    from synth.device import fill_inputs, fill_mha
    D = dsa.dsa
    wl = W.WORKLOADS["p4k"]
    d = fill_inputs(wl)
    m = fill_mha(wl)
    dn, dr, dvh = W.mha_dims(wl)
    dims = D.Dims.of(wl)
    B, T, S, k, H = wl.batch, wl.n_q, wl.n_kv, wl.topk, wl.heads
    st = stream.cuda_stream
    iargs = (d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"])
    out = torch.empty((B, T, H, dvh), dtype=torch.int16, device="cuda")
    lse = torch.empty((B, T, H), dtype=torch.float32, device="cuda")
    nws = D.dsa_masked_mha_workspace_size(dims, dn, dvh)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    t = Timer(torch, stream)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = t.start()
        for _ in range(reps):
            fn()
        e1 = t.event()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    masked_ms = timed(lambda: D.dsa_masked_mha_forward(dims, dn, dvh, *iargs, m["q_mha"], d["kv"], m["w_uk"],
                                                       m["w_uv"], wl.sm_scale, out, lse, None, ws, nws, stream=st))
    dims_f, out_f, lse_f, fws, nfws = alloc_forward(torch, wl, dsa)
    sparse_ms = timed(lambda: D.dsa_forward(dims_f, *iargs, d["q"], d["kv"], wl.sm_scale, out_f, lse_f, None, fws,
                                            nfws, stream=st))
    del out_f, lse_f, fws
    # stages of the masked path
    sc = torch.empty((B, T, S), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, T, k), dtype=torch.int32, device="cuda")
    mask = torch.empty((B, (S + 31) // 32, T), dtype=torch.int32, device="cuda")
    k_mha = torch.empty((B, H, S, dn), dtype=torch.int16, device="cuda")
    v_mha = torch.empty((B, H, S, dvh), dtype=torch.int16, device="cuda")
    calls = {
        "indexer": lambda: D.dsa_indexer_scores(dims, *iargs, sc, S, stream=st),
        "topk": lambda: D.dsa_topk(dims, sc, S, idx, stream=st),
        "selection_mask": lambda: D.dsa_selection_mask(dims, idx, mask, stream=st),
        "decompress": lambda: D.dsa_mha_decompress(dims, dn, dvh, d["kv"], m["w_uk"], m["w_uv"], S, k_mha, v_mha,
                                                   stream=st),
        "masked_attention": lambda: D.dsa_masked_mha_attn(dims, dn, dvh, m["q_mha"], d["kv"], k_mha, v_mha, mask,
                                                          wl.sm_scale, out, lse, stream=st),
    }
    for f in calls.values():
        f()
    torch.cuda.synchronize()
    tot = {name: 0.0 for name in calls}
    for _ in range(reps):
        ev = [t.start()]
        for f in calls.values():
            f()
            ev.append(t.event())
        torch.cuda.synchronize()
        for j, name in enumerate(calls):
            tot[name] += ev[j].elapsed_time(ev[j + 1]) / reps
    attn_flop = 2.0 * wl.causal_pairs() * H * (dn + dr + dvh)
    dec_flop = 2.0 * B * S * wl.dim_v * H * (dn + dvh)
    attn_tf = attn_flop / (tot["masked_attention"] / 1e3) / 1e12
    dec_tf = dec_flop / (tot["decompress"] / 1e3) / 1e12
    res = {"workload": "p4k: 1 x 4096 prefill, k = 2048, 128 heads; MHA heads 128 + 64 rope, values 128",
           "masked_mha_ms": masked_ms, "sparse_mqa_ms": sparse_ms, "speedup_vs_sparse": sparse_ms / masked_ms,
           "masked_query_tokens_per_s": B * T / (masked_ms / 1e3), "stages_ms": tot,
           "masked_attention_tflops": attn_tf, "masked_attention_frac": attn_tf / PEAK_BF16_TFLOPS,
           "masked_attention_flop": attn_flop,
           "decompress_tflops": dec_tf, "decompress_frac": dec_tf / PEAK_BF16_TFLOPS, "decompress_flop": dec_flop}
    del d, m, ws, sc, k_mha, v_mha
    return res


def roofline_sum(wl, ms):
    """Lower bound on the forward step from the three stages' rooflines:
    indexer FP8 work, top-k bytes, and the larger of the attention's BF16
    work and its q/out bytes, at the published peaks."""
    P, Q = wl.causal_pairs(), wl.selected_pairs()
    L = wl.batch * wl.n_q
    t_idx = 2.0 * P * wl.idx_heads * wl.idx_dim / (PEAK_FP8_TFLOPS * 1e12)
    t_topk = (4.0 * P + 4.0 * L * wl.topk) / (PEAK_HBM_GBS * 1e9)
    qo_bytes = 2.0 * L * wl.heads * (wl.dim_qk + wl.dim_v)
    t_attn = max(2.0 * Q * wl.heads * (wl.dim_qk + wl.dim_v) / (PEAK_BF16_TFLOPS * 1e12), qo_bytes / (PEAK_HBM_GBS * 1e9))
    t_star = (t_idx + t_topk + t_attn) * 1e3
    return {"t_star_ms": t_star, "indexer_ms": t_idx * 1e3, "topk_ms": t_topk * 1e3, "attention_ms": t_attn * 1e3,
            "frac": t_star / ms, "query_tokens_per_s_at_roof": L / (t_star / 1e3)}


def hbm_copy_rate(torch, mib=1024, reps=5):
    """Achievable HBM rate on this machine: a plain device-to-device copy of
    `mib` MiB (read + write bytes per second)."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * n / (e0.elapsed_time(e1) / reps / 1e3) / 1e9
    del src, dst
    return {"GB_per_s": gbs, "frac_of_hbm_peak": gbs / PEAK_HBM_GBS, "bytes_copied": n}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def stratified(L, n_rows):
    return [int((r + 0.5) * L / n_rows) for r in range(n_rows)]


def cpu_baseline(wl, n_rows, gpu_sel=None):
    """The CPU oracle (unchanged) on a stratified sample of query rows
    floor((r + 1/2) L / R), each stage timed separately.  Input generation is
    not timed.  With gpu_sel (the GPU's selection of those rows), also the
    set recall R_k = |T_k n S_k| / k of the GPU set against the oracle set
    (Sec. 5, Eq. (14)) and the oracle's cutoff margin s_(k) - s_(k+1)
    (Sec. 5.2, Eq. (18)) over the sampled rows."""
    from oracle import dsa_oracle as O
    from synth import workloads as W
    rows = stratified(wl.n_q, n_rows)
    c, s = W.k_idx_fp8(wl, 0, 0, wl.n_kv)
    k_all = O.dequant_e4m3(c, s)
    kv = O.bf16_decode(W.kv_bf16_rows(wl, 0, np.arange(wl.n_kv)))
    qc, qs = W.q_idx_fp8(wl, 0, rows)
    qi = O.dequant_e4m3(qc, qs)
    w = O.bf16_decode(W.w_idx_bf16(wl, 0, rows))
    q = O.bf16_decode(W.q_bf16(wl, 0, rows))
    st = {"indexer": 0.0, "topk": 0.0, "attention": 0.0}
    recall, margins = [], []
    for n, i in enumerate(rows):
        p = wl.q_pos0 + i
        t0 = time.perf_counter()
        sc = O.indexer_row(qi[n], w[n], k_all, p)
        t1 = time.perf_counter()
        sel = O.topk_row(sc, wl.topk)
        t2 = time.perf_counter()
        O.sparse_mla_row(q[n], kv, sel, wl.sm_scale, wl.dim_v)
        t3 = time.perf_counter()
        st["indexer"] += t1 - t0
        st["topk"] += t2 - t1
        st["attention"] += t3 - t2
        if gpu_sel is not None and sc.size > wl.topk:
            ref = sel[sel >= 0]
            g = gpu_sel[n][gpu_sel[n] >= 0]
            recall.append(np.intersect1d(ref, g).size / ref.size)
            srt = np.sort(sc.astype(np.float64))[::-1]
            margins.append(float(srt[wl.topk - 1] - srt[wl.topk]))
    dt = sum(st.values())
    res = {"value": n_rows / dt, "unit": "query-tokens/s", "cores": int(blas_threads()), "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{n_rows} stratified query rows of {wl.name} (rows floor((r+1/2)L/{n_rows})), "
                     f"float64 numpy, {dt:.1f} s timed; input generation excluded",
           "stage_s": st}
    if recall:
        m = np.array(margins)
        edges = [0.0, 1e-6, 1e-5, 1e-4, 1e-3, 1e-2, 1e-1, np.inf]
        res["selection_vs_oracle"] = {
            "rows": len(recall), "recall_mean": float(np.mean(recall)), "recall_min": float(np.min(recall)),
            "margin_quantiles": {str(qq): float(np.quantile(m, qq)) for qq in (0.0, 0.01, 0.5, 0.99)},
            "margin_hist": {f"[{a:g},{b:g})": int(x) for a, b, x in zip(edges[:-1], edges[1:],
                                                                         np.histogram(m, edges)[0])}}
    return res


def cpu_baseline_decode(dw, n_seq):
    """The CPU oracle on the first n_seq sequences of the decode step (one
    query row each against its own 128K cache), each stage timed."""
    from oracle import dsa_oracle as O
    from synth import workloads as W
    st = {"indexer": 0.0, "topk": 0.0, "attention": 0.0}
    for b in range(n_seq):
        c, s = W.k_idx_fp8(dw, b, 0, dw.n_kv)
        k_all = O.dequant_e4m3(c, s)
        qc, qs = W.q_idx_fp8(dw, b, [0])
        qi = O.dequant_e4m3(qc, qs)[0]
        w = O.bf16_decode(W.w_idx_bf16(dw, b, [0]))[0]
        q = O.bf16_decode(W.q_bf16(dw, b, [0]))[0]
        t0 = time.perf_counter()
        sc = O.indexer_row(qi, w, k_all, dw.q_pos0)
        t1 = time.perf_counter()
        sel = O.topk_row(sc, dw.topk)
        t2 = time.perf_counter()
        kv = O.bf16_decode(W.kv_bf16_rows(dw, b, sel))
        t2b = time.perf_counter()
        O.sparse_mla_row(q, kv, np.arange(sel.size), dw.sm_scale, dw.dim_v)
        t3 = time.perf_counter()
        st["indexer"] += t1 - t0
        st["topk"] += t2 - t1
        st["attention"] += t3 - t2b
    dt = sum(st.values())
    return {"value": n_seq / dt, "unit": "decode query-tokens/s", "cores": int(blas_threads()), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{n_seq} of the 64 sequences of {dw.name} (one query row each), float64 numpy, "
                      f"{dt:.2f} s timed; input generation and the selected rows' generation excluded",
            "stage_s": st}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="p128k")
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="stratified query rows the CPU oracle baseline times (1024: about 10 s on 16 threads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-decode-seqs", type=int, default=2,
                    help="decode sequences the CPU oracle times per stage (each regenerates its 128K key cache)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=1)
    ap.add_argument("--short-prefill-only", action="store_true",
                    help="run only the short-prefill comparison (4K tokens: masked MHA mode vs sparse MQA) "
                         "and print its JSON; for profiling those kernels alone")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a known-size kernel that "
                         "calibrates FETCH_SIZE/WRITE_SIZE counters in a rocprofv3 --pmc run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the DSA forward path here is a single-GPU build "
              "(multi-GPU sharding is a design note, not implemented); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_long_amd as dsa
    from synth import workloads as W
    from synth.device import fill_inputs

    wl = W.WORKLOADS[args.workload]
    stream = torch.cuda.current_stream()
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {n} bytes done")
        del src, dst
    if args.short_prefill_only:
        print(json.dumps({"short_prefill": time_short_prefill(torch, dsa, stream, reps=max(args.steps, 1),
                                                              warmup=args.warmup)}), flush=True)
        return
    log(f"[bench] filling {wl.name} inputs on the GPU")
    d = fill_inputs(wl)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} dsa_forward steps after {args.warmup} warm-up")
    ms = time_forward(torch, wl, d, dsa, args.steps, args.warmup, stream)
    toks = wl.batch * wl.n_q / (ms / 1e3)
    log(f"[bench] dsa_forward {ms:.2f} ms/step -> {toks:,.0f} query-tokens/s")

    log("[bench] per-stage pass (indexer / top-k / attention events)")
    stages, launches, _ = time_stages(torch, wl, d, dsa, args.stage_reps, stream)
    idx_flop = wl.indexer_flop()
    attn_flop = wl.attn_flop()
    idx_tflops = idx_flop / (stages["indexer"] / 1e3) / 1e12
    attn_tflops = attn_flop / (stages["attention"] / 1e3) / 1e12
    topk_bytes = 4.0 * wl.causal_pairs() + 4.0 * wl.batch * wl.n_q * wl.topk
    topk_gbs = topk_bytes / (stages["topk"] / 1e3) / 1e9
    log(f"[bench] stages ms {stages}; indexer {idx_tflops:.1f} TFLOP/s, attention {attn_tflops:.1f} TFLOP/s, "
        f"top-k {topk_gbs:.0f} GB/s")
    dom = max(stages, key=stages.get)
    kname = STAGE_KERNELS[dom][0]
    if dom == "indexer":
        roof = {"kernel": kname, "bound": "mfma", "achieved": idx_tflops,
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "dtype": "fp8"}
    elif dom == "attention":
        roof = {"kernel": kname, "bound": "mfma", "achieved": attn_tflops,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "dtype": "bf16"}
    else:
        roof = {"kernel": kname, "bound": "hbm", "achieved": topk_gbs, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) from profiles/, or null
    roof["traffic"] = profiled_traffic(dom, wl.name)
    roof["launches"] = launches
    roof["avg_launch_us"] = stages[dom] * 1e3 / max(launches, 1)

    gpu_sel = None
    if not args.no_cpu_baseline:
        # the GPU's selection of the rows the CPU oracle samples (an untimed forward with idx_out)
        dims, out, lse, ws, nws = alloc_forward(torch, wl, dsa)
        idx_all = torch.empty((wl.batch, wl.n_q, wl.topk), dtype=torch.int32, device="cuda")
        dsa.dsa_forward(dims, d["q_idx"], d["q_scale"], d["w_idx"], d["k_idx"], d["k_scale"], d["q"], d["kv"],
                        wl.sm_scale, out, lse, idx_all, ws, nws, stream=stream.cuda_stream)
        torch.cuda.synchronize()
        gpu_sel = idx_all[0, stratified(wl.n_q, args.cpu_rows)].cpu().numpy()
        del dims, out, lse, ws, idx_all
        torch.cuda.empty_cache()

    train = None
    if not args.no_decode:
        log("[bench] sparse-stage training forward (dsa_forward_kl)")
        kms, kl_mean = time_forward_kl(torch, wl, d, dsa, max(1, min(args.steps, 2)), 1, stream)
        kl_ms = kms - ms
        qk_flop = 2.0 * wl.selected_pairs() * wl.heads * wl.dim_qk
        train = {"ms_per_step": kms, "query_tokens_per_s": wl.batch * wl.n_q / (kms / 1e3),
                 "kl_increment_ms": kl_ms, "kl_qk_tflops": qk_flop / (kl_ms / 1e3) / 1e12 if kl_ms > 0 else None,
                 "mean_kl": kl_mean}
        log(f"[bench] training forward {train}")
    del d
    torch.cuda.empty_cache()

    p32k = None
    if not args.no_decode and wl.name != "p32k":
        pw = W.WORKLOADS["p32k"]
        log("[bench] prefill p32k (low-rank latents)")
        pd = fill_inputs(pw)
        torch.cuda.synchronize()
        pms = time_forward(torch, pw, pd, dsa, max(args.steps, 3), 1, stream)
        pst, _, _ = time_stages(torch, pw, pd, dsa, 1, stream)
        p32k = {"workload": "p32k", "ms_per_step": pms, "query_tokens_per_s": pw.n_q / (pms / 1e3),
                "stages_ms": pst,
                "indexer_fp8_tflops": pw.indexer_flop() / (pst["indexer"] / 1e3) / 1e12,
                "attention_bf16_tflops": pw.attn_flop() / (pst["attention"] / 1e3) / 1e12,
                "topk_GB_per_s": (4.0 * pw.causal_pairs() + 4.0 * pw.n_q * pw.topk) / (pst["topk"] / 1e3) / 1e9,
                "roofline_sum": roofline_sum(pw, pms)}
        log(f"[bench] p32k {p32k}")
        del pd
        torch.cuda.empty_cache()

    decode = None
    if not args.no_decode:
        dw = W.WORKLOADS["dec64"]
        log("[bench] decode workload dec64")
        dd = fill_inputs(dw)
        torch.cuda.synchronize()
        dms = time_forward(torch, dw, dd, dsa, max(args.steps, 10), args.warmup, stream)
        dstages, _, _ = time_stages(torch, dw, dd, dsa, 10, stream)
        B, S, k = dw.batch, dw.n_kv, dw.topk
        idx_bytes = B * S * (dw.idx_dim + 4) + B * dw.idx_heads * (dw.idx_dim + 2) + B * 4 + 4 * B * S
        topk_b = 4 * B * S + 4 * B * k
        mla_bytes = B * k * dw.dim_qk * 2 + B * dw.heads * dw.dim_qk * 2 + B * dw.heads * dw.dim_v * 2
        step_bytes = idx_bytes + topk_b + mla_bytes
        decode = {"workload": "dec64", "ms_per_step": dms, "GB_per_s": step_bytes / (dms / 1e3) / 1e9,
                  "stages_ms": dstages,
                  "indexer_GB_per_s": idx_bytes / (dstages["indexer"] / 1e3) / 1e9,
                  "topk_GB_per_s": topk_b / (dstages["topk"] / 1e3) / 1e9,
                  "mla_gather_GB_per_s": mla_bytes / (dstages["attention"] / 1e3) / 1e9,
                  "algorithmic_bytes_per_step": step_bytes}
        decode["mla_frac_of_hbm_peak"] = decode["mla_gather_GB_per_s"] / PEAK_HBM_GBS
        decode["plan"] = {"topk_parts": int(dsa.dsa.dsa_forward_plan_of(dsa.Dims.of(dw)).topk_parts),
                          "attn_splits": int(dsa.dsa.dsa_forward_plan_of(dsa.Dims.of(dw)).attn_splits)}
        log(f"[bench] decode {dms*1e3:.1f} us/step; {decode}")
        del dd
        torch.cuda.empty_cache()

    decode_paged = None
    if not args.no_decode:
        log("[bench] paged variable-length decode (dec64 layout, 64-token pages)")
        decode_paged = time_decode_paged(torch, dsa, stream)
        log(f"[bench] decode paged {decode_paged}")
        torch.cuda.empty_cache()

    quant = None
    if not args.no_decode:
        log("[bench] FP8 quantisation of the index keys and of 16384 query tokens")
        quant = time_quantize(torch, dsa, wl, stream)
        log(f"[bench] quantise {quant}")
        torch.cuda.empty_cache()

    short = None
    if not args.no_decode:
        log("[bench] short prefill p4k: sparse MQA forward vs masked MHA mode")
        short = time_short_prefill(torch, dsa, stream)
        log(f"[bench] short prefill {short}")
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline on {args.cpu_rows} rows")
        cpu = cpu_baseline(wl, args.cpu_rows, gpu_sel)
        log(f"[bench] cpu {cpu}")
        if not args.no_decode and args.cpu_decode_seqs > 0:
            cpu["decode"] = cpu_baseline_decode(W.WORKLOADS["dec64"], args.cpu_decode_seqs)
            log(f"[bench] cpu decode {cpu['decode']}")

    res = {
        "metric": METRIC, "value": toks, "unit": "query-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8/bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "L": wl.n_kv, "n_q": wl.n_q, "topk": wl.topk,
                   "idx_heads": wl.idx_heads, "idx_dim": wl.idx_dim, "heads": wl.heads, "dim_qk": wl.dim_qk,
                   "dim_v": wl.dim_v},
        "stages_ms": stages, "indexer_fp8_tflops": idx_tflops, "attention_bf16_tflops": attn_tflops,
        "topk_GB_per_s": topk_gbs, "roofline": roof, "train_forward_kl": train, "decode": decode,
        "p32k": p32k, "decode_paged": decode_paged, "short_prefill": short,
        "quantize": quant, "cpu_baseline": cpu, "roofline_sum": roofline_sum(wl, ms),
        "hbm_copy": hbm_copy_rate(torch),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
