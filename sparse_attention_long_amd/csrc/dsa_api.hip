// C ABI of the DSA forward path: argument validation, workspace planning and
// kernel dispatch.  Every check runs on the host before the first HIP call,
// so invalid calls leave outputs untouched and launch nothing.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/dsa.h"
#include "dsa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return DSA_OK;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

int check_common(const dsa_dims* d) {
  REQUIRE(d != nullptr, DSA_ERR_INVALID_ARG, "dims is NULL");
  REQUIRE(d->batch >= 1 && d->n_q >= 1 && d->n_kv >= 1, DSA_ERR_INVALID_ARG,
          "batch, n_q and n_kv must be >= 1 (got %d, %d, %d)", d->batch, d->n_q, d->n_kv);
  REQUIRE(d->q_pos0 >= 0, DSA_ERR_INVALID_ARG, "q_pos0 must be >= 0 (got %d)", d->q_pos0);
  REQUIRE((int64_t)d->q_pos0 + d->n_q <= d->n_kv, DSA_ERR_INVALID_ARG,
          "query positions q_pos0 + n_q (%lld) exceed n_kv (%d)", (long long)d->q_pos0 + d->n_q, d->n_kv);
  REQUIRE(d->topk >= 1 && d->topk <= 2048, DSA_ERR_UNSUPPORTED, "topk must be in [1, 2048] (got %d)", d->topk);
  REQUIRE((int64_t)d->batch * d->n_q <= (1ll << 30), DSA_ERR_UNSUPPORTED, "batch * n_q too large");
  return DSA_OK;
}

int check_indexer_dims(const dsa_dims* d) {
  REQUIRE(d->idx_heads >= 1 && d->idx_heads <= 64, DSA_ERR_UNSUPPORTED,
          "idx_heads must be in [1, 64] (got %d)", d->idx_heads);
  REQUIRE(d->idx_dim >= 16 && d->idx_dim <= 128 && d->idx_dim % 16 == 0, DSA_ERR_UNSUPPORTED,
          "idx_dim must be a multiple of 16 in [16, 128] (got %d)", d->idx_dim);
  return DSA_OK;
}

int check_attn_dims(const dsa_dims* d) {
  REQUIRE(d->heads >= 1 && d->dim_qk >= 1 && d->dim_v >= 1 && d->dim_v <= d->dim_qk, DSA_ERR_INVALID_ARG,
          "heads/dim_qk/dim_v inconsistent (%d, %d, %d)", d->heads, d->dim_qk, d->dim_v);
  REQUIRE(dsa::attn_dims_supported(d->heads, d->dim_qk, d->dim_v), DSA_ERR_UNSUPPORTED,
          "attention dims (heads %d, dim_qk %d, dim_v %d) not built; supported: dim_qk 576 / dim_v 512 "
          "with heads <= 128, dim_qk 80 / dim_v 64 with heads <= 32",
          d->heads, d->dim_qk, d->dim_v);
  return DSA_OK;
}

// Dense caches: the row gathers address a sequence's latent cache with
// 32-bit byte offsets (page pools use 64-bit row addresses).
int check_dense_kv_size(const dsa_dims* d) {
  REQUIRE((uint64_t)d->n_kv * (uint64_t)d->dim_qk * 2u < (1ull << 32), DSA_ERR_UNSUPPORTED,
          "one sequence's latent cache (n_kv %d x dim_qk %d bf16) must be below 4 GiB", d->n_kv, d->dim_qk);
  return DSA_OK;
}

// Paged / variable-length layout: host checks of the descriptor (the device
// arrays themselves are clamped by the kernels).  Fills `pk`.
int check_paged(const dsa_dims* d, const dsa_paged_kv* p, dsa::PagedKV* pk) {
  REQUIRE(p != nullptr, DSA_ERR_INVALID_ARG, "paged layout is NULL");
  REQUIRE(p->seq_lens != nullptr && aligned(p->seq_lens, 4), DSA_ERR_INVALID_ARG,
          "seq_lens must be a non-null, 4-byte aligned device pointer");
  *pk = dsa::PagedKV{};
  pk->seq_lens = p->seq_lens;
  pk->n_q_total = d->n_q;
  if (p->page_table) {
    REQUIRE(aligned(p->page_table, 4), DSA_ERR_INVALID_ARG, "page_table must be 4-byte aligned");
    REQUIRE(p->page_size >= 64 && p->page_size % 64 == 0, DSA_ERR_UNSUPPORTED,
            "page_size must be a positive multiple of 64 (got %d)", p->page_size);
    REQUIRE((int64_t)p->max_pages * p->page_size >= d->n_kv, DSA_ERR_INVALID_ARG,
            "max_pages (%d) x page_size (%d) must cover n_kv (%d)", p->max_pages, p->page_size, d->n_kv);
    REQUIRE(p->num_pages >= 1 && (int64_t)p->num_pages * p->page_size < (1ll << 31), DSA_ERR_UNSUPPORTED,
            "num_pages (%d) x page_size (%d) must be in [1, 2^31)", p->num_pages, p->page_size);
    pk->page_table = p->page_table;
    pk->page_size = p->page_size;
    pk->max_pages = p->max_pages;
    pk->num_pages = p->num_pages;
  }
  return DSA_OK;
}

// dims for the paged calls: positions come from seq_lens, so q_pos0 plays no
// part (set to 0 for the common checks).
dsa_dims paged_dims(const dsa_dims* d) {
  dsa_dims dd = *d;
  dd.q_pos0 = 0;
  return dd;
}

// Split of the selected slots across workgroups for attention: enough
// workgroups to cover the 256 compute units, at least 128 slots per split.
int attn_nsplit(const dsa_dims* d) {
  const int64_t rows = (int64_t)d->batch * d->n_q;
  if (rows >= 256) return 1;
  int ns = (int)((256 + rows - 1) / rows);
  const int max_ns = (d->topk + 127) / 128;
  if (ns > max_ns) ns = max_ns;
  if (ns > 16) ns = 16;
  return ns < 1 ? 1 : ns;
}

size_t attn_partial_bytes(const dsa_dims* d, int64_t rows_per_seq) {
  const int ns = attn_nsplit(d);
  if (ns <= 1) return 0;
  // bf16 partial outputs, then one f32 log-sum-exp per (row, split, head)
  const size_t n = (size_t)d->batch * rows_per_seq * ns * d->heads;
  return (n * d->dim_v * sizeof(uint16_t) + 15) / 16 * 16 + n * sizeof(float);
}

// Query rows per chunk of dsa_forward: a chunk's scores take about 256 MiB
// of the workspace (512 rows at 128K keys), written by the indexer and read
// back by top-k while they are still largely in the 256 MB Infinity Cache.
// Measured per 128K prefill step with one stream: 220, 147, 142, 146 and
// 151 ms for 64, 128, 256, 512 and 1024 MiB per chunk.
int64_t forward_chunk_rows(const dsa_dims* d) {
  const int64_t budget = 256ll << 20;
  int64_t tc = budget / ((int64_t)d->batch * d->n_kv * 4);
  if (tc >= 64) tc = tc / 32 * 32;
  if (tc > 1) tc &= ~(int64_t)1;   // even: a row keeps its indexer slot parity in every chunk
  if (tc < 1) tc = 1;
  if (tc > d->n_q) tc = d->n_q;
  return tc;
}

// A chunk's buffers: scores, selection, attention partials and (for a few
// long rows) the top-k parts' candidate lists, each 256-byte aligned.
struct ForwardLayout {
  int64_t tc;
  int topk_parts;   // top-k workgroups per row (1: one per row)
  int attn_splits;  // attention workgroups per row (1: no partials, no combine)
  size_t scores_off, idx_off, part_off, topk_off, total;
};

ForwardLayout forward_layout(const dsa_dims* d) {
  ForwardLayout L;
  L.tc = forward_chunk_rows(d);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  L.scores_off = 0;
  L.idx_off = up((size_t)d->batch * L.tc * d->n_kv * sizeof(float));
  L.part_off = L.idx_off + up((size_t)d->batch * L.tc * d->topk * sizeof(int32_t));
  L.topk_off = L.part_off + up(attn_partial_bytes(d, L.tc));
  L.topk_parts = dsa::topk_split_parts((int64_t)d->batch * L.tc, d->n_kv);
  L.attn_splits = attn_nsplit(d);
  L.total = L.topk_off + up(dsa::topk_split_bytes((int64_t)d->batch * L.tc, L.topk_parts));
  return L;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

dsa::IndexerArgs indexer_args(const dsa_dims* d, const uint8_t* q_idx, const float* q_scale, const uint16_t* w,
                              const uint8_t* k_idx, const float* k_scale, float* scores, int64_t ld,
                              int64_t i0, int rows, int64_t sc_rows_b, const dsa::PagedKV& pk) {
  dsa::IndexerArgs a{};
  a.pk = pk;
  a.q_idx = q_idx + i0 * d->idx_heads * d->idx_dim;
  a.q_scale = q_scale + i0;
  a.w = w + i0 * d->idx_heads;
  a.k_idx = k_idx;
  a.k_scale = k_scale;
  a.scores = scores;
  a.ld = ld;
  a.qrows_b = d->n_q;
  a.sc_rows_b = sc_rows_b;
  a.B = d->batch;
  a.rows = rows;
  a.pos0 = (pk.seq_lens ? 0 : d->q_pos0) + (int)i0;
  a.S = d->n_kv;
  a.HI = d->idx_heads;
  a.dI = d->idx_dim;
  return a;
}

}  // namespace

extern "C" {

int dsa_version(void) { return 200; }

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported dimensions";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {

int indexer_impl(const dsa_dims* d, const dsa::PagedKV& pk, const uint8_t* q_idx, const float* q_scale,
                 const uint16_t* w_idx, const uint8_t* k_idx, const float* k_scale, float* scores, int64_t ld,
                 void* stream) {
  int st;
  if ((st = check_common(d)) != DSA_OK) return st;
  if ((st = check_indexer_dims(d)) != DSA_OK) return st;
  REQUIRE(q_idx && q_scale && w_idx && k_idx && k_scale && scores, DSA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned(q_idx, 16) && aligned(k_idx, 16), DSA_ERR_INVALID_ARG, "q_idx and k_idx must be 16-byte aligned");
  REQUIRE(aligned(q_scale, 4) && aligned(k_scale, 4) && aligned(scores, 4) && aligned(w_idx, 2),
          DSA_ERR_INVALID_ARG, "misaligned scale/score/weight pointer");
  REQUIRE(ld >= d->n_kv, DSA_ERR_INVALID_ARG, "ld (%lld) must be >= n_kv (%d)", (long long)ld, d->n_kv);
  const dsa::IndexerArgs a =
      indexer_args(d, q_idx, q_scale, w_idx, k_idx, k_scale, scores, ld, 0, d->n_q, d->n_q, pk);
  return hip_status(dsa::launch_indexer(a, d->n_q <= dsa::kIndexerDecodeMaxRows, (hipStream_t)stream),
                    "indexer launch");
}

// Top-k parts per row of a standalone call with a workspace (the rule the
// forward applies to its chunks).
int topk_call_parts(const dsa_dims* d) { return dsa::topk_split_parts((int64_t)d->batch * d->n_q, d->n_kv); }

int topk_impl(const dsa_dims* d, const dsa::PagedKV& pk, const float* scores, int64_t ld, int32_t* idx,
              void* stream, void* ws = nullptr, size_t ws_bytes = 0, bool use_ws = false) {
  int st;
  if ((st = check_common(d)) != DSA_OK) return st;
  REQUIRE(scores && idx, DSA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned(scores, 4) && aligned(idx, 4), DSA_ERR_INVALID_ARG, "misaligned scores/idx pointer");
  REQUIRE(ld >= d->n_kv, DSA_ERR_INVALID_ARG, "ld (%lld) must be >= n_kv (%d)", (long long)ld, d->n_kv);
  REQUIRE(d->n_kv <= dsa::topk_max_kv(), DSA_ERR_UNSUPPORTED, "n_kv (%d) exceeds the top-k limit %d", d->n_kv,
          dsa::topk_max_kv());
  dsa::TopkArgs a{};
  a.pk = pk;
  a.scores = scores;
  a.idx = idx;
  a.ld = ld;
  a.sc_rows_b = d->n_q;
  a.idx_rows_b = d->n_q;
  a.B = d->batch;
  a.rows = d->n_q;
  a.pos0 = pk.seq_lens ? 0 : d->q_pos0;
  a.S = d->n_kv;
  a.k = d->topk;
  if (use_ws) {
    const int parts = topk_call_parts(d);
    const size_t need = dsa::topk_split_bytes((int64_t)d->batch * d->n_q, parts);
    REQUIRE(need == 0 || (ws != nullptr && ws_bytes >= need), DSA_ERR_WORKSPACE,
            "top-k needs %zu workspace bytes (got %zu)", need, ws ? ws_bytes : (size_t)0);
    REQUIRE(need == 0 || aligned(ws, 256), DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    return hip_status(dsa::launch_topk_split(a, parts, ws, (hipStream_t)stream), "top-k launch");
  }
  return hip_status(dsa::launch_topk(a, (hipStream_t)stream), "top-k launch");
}

int validate_attn(const dsa_dims* d, const uint16_t* q, const uint16_t* kv, const int32_t* idx, float sm_scale,
                  const uint16_t* out, const float* lse, bool idx_required, bool dense) {
  int st;
  if ((st = check_common(d)) != DSA_OK) return st;
  if ((st = check_attn_dims(d)) != DSA_OK) return st;
  if (dense && (st = check_dense_kv_size(d)) != DSA_OK) return st;
  REQUIRE(q && kv && out && (idx || !idx_required), DSA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned(q, 16) && aligned(kv, 16) && aligned(out, 16) && aligned(idx, 4) && aligned(lse, 4),
          DSA_ERR_INVALID_ARG, "q, kv and out must be 16-byte aligned; idx and lse 4-byte aligned");
  REQUIRE(std::isfinite(sm_scale) && sm_scale > 0.f, DSA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  return DSA_OK;
}

int attn_impl(const dsa_dims* d, const dsa::PagedKV& pk, const uint16_t* q, const uint16_t* kv,
              const int32_t* idx, float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
              void* stream) {
  int st;
  if ((st = validate_attn(d, q, kv, idx, sm_scale, out, lse, true, pk.page_table == nullptr)) != DSA_OK) return st;
  const size_t need = attn_partial_bytes(d, d->n_q);
  REQUIRE(need == 0 || (ws != nullptr && ws_bytes >= need), DSA_ERR_WORKSPACE,
          "attention needs %zu workspace bytes (got %zu)", need, ws ? ws_bytes : (size_t)0);
  REQUIRE(need == 0 || aligned(ws, 16), DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  dsa::AttnArgs a{};
  a.pk = pk;
  a.q = q;
  a.kv = kv;
  a.idx = idx;
  a.out = out;
  a.lse = lse;
  a.nsplit = attn_nsplit(d);
  const size_t rows_total = (size_t)d->batch * d->n_q;
  a.part_o = (uint16_t*)ws;
  a.part_lse = a.nsplit > 1
                   ? (float*)((char*)ws + (rows_total * a.nsplit * d->heads * d->dim_v * sizeof(uint16_t) + 15) / 16 * 16)
                   : nullptr;
  a.qrows_b = d->n_q;
  a.idx_rows_b = d->n_q;
  a.B = d->batch;
  a.rows = d->n_q;
  a.S = d->n_kv;
  a.H = d->heads;
  a.Dk = d->dim_qk;
  a.Dv = d->dim_v;
  a.k = d->topk;
  a.sm_scale = sm_scale;
  return hip_status(dsa::launch_sparse_mla(a, (hipStream_t)stream), "attention launch");
}

int forward_impl(const dsa_dims* d, const dsa::PagedKV& pk, const uint8_t* q_idx, const float* q_scale,
                 const uint16_t* w_idx, const uint8_t* k_idx, const float* k_scale, const uint16_t* q,
                 const uint16_t* kv, float sm_scale, uint16_t* out, float* lse, int32_t* idx_out, void* ws,
                 size_t ws_bytes, void* stream, float* kl = nullptr) {
  int st;
  REQUIRE(kl == nullptr || (lse != nullptr && aligned(kl, 4)), DSA_ERR_INVALID_ARG,
          "the indexer KL needs lse (the attention's log-sum-exp) and a 4-byte aligned kl buffer");
  if ((st = validate_attn(d, q, kv, idx_out, sm_scale, out, lse, false, pk.page_table == nullptr)) != DSA_OK)
    return st;
  if ((st = check_indexer_dims(d)) != DSA_OK) return st;
  REQUIRE(q_idx && q_scale && w_idx && k_idx && k_scale, DSA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned(q_idx, 16) && aligned(k_idx, 16), DSA_ERR_INVALID_ARG, "q_idx and k_idx must be 16-byte aligned");
  REQUIRE(aligned(q_scale, 4) && aligned(k_scale, 4) && aligned(w_idx, 2), DSA_ERR_INVALID_ARG,
          "misaligned scale/weight pointer");
  REQUIRE(d->n_kv <= dsa::topk_max_kv(), DSA_ERR_UNSUPPORTED, "n_kv (%d) exceeds the top-k limit %d", d->n_kv,
          dsa::topk_max_kv());
  const ForwardLayout L = forward_layout(d);
  REQUIRE(ws != nullptr && ws_bytes >= L.total, DSA_ERR_WORKSPACE, "forward needs %zu workspace bytes (got %zu)",
          L.total, ws ? ws_bytes : (size_t)0);
  REQUIRE(aligned(ws, 256), DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

  const hipStream_t s = (hipStream_t)stream;
  const bool decode_form = d->n_q <= dsa::kIndexerDecodeMaxRows;
  const int nsplit = L.attn_splits;
  const int pos_base = pk.seq_lens ? 0 : d->q_pos0;
  char* wsb = (char*)ws;
  float* sc = (float*)(wsb + L.scores_off);
  for (int64_t i0 = 0; i0 < d->n_q; i0 += L.tc) {
    const int rows = (int)((d->n_q - i0) < L.tc ? (d->n_q - i0) : L.tc);
    const dsa::IndexerArgs ia =
        indexer_args(d, q_idx, q_scale, w_idx, k_idx, k_scale, sc, d->n_kv, i0, rows, L.tc, pk);
    hipError_t e = dsa::launch_indexer(ia, decode_form, s);
    if (e != hipSuccess) return hip_status(e, "indexer launch");

    dsa::TopkArgs ta{};
    ta.pk = pk;
    ta.scores = sc;
    ta.ld = d->n_kv;
    ta.sc_rows_b = L.tc;
    ta.idx = idx_out ? idx_out + i0 * d->topk : (int32_t*)(wsb + L.idx_off);
    ta.idx_rows_b = idx_out ? d->n_q : L.tc;
    ta.B = d->batch;
    ta.rows = rows;
    ta.pos0 = pos_base + (int)i0;
    ta.S = d->n_kv;
    ta.k = d->topk;
    e = dsa::launch_topk_split(ta, L.topk_parts, wsb + L.topk_off, s);
    if (e != hipSuccess) return hip_status(e, "top-k launch");

    dsa::AttnArgs aa{};
    aa.pk = pk;
    aa.q = q + i0 * d->heads * d->dim_qk;
    aa.kv = kv;
    aa.idx = ta.idx;
    aa.idx_rows_b = ta.idx_rows_b;
    aa.out = out + i0 * d->heads * d->dim_v;
    aa.lse = lse ? lse + i0 * d->heads : nullptr;
    aa.nsplit = nsplit;
    aa.part_o = (uint16_t*)(wsb + L.part_off);
    aa.part_lse =
        nsplit > 1
            ? (float*)((char*)aa.part_o + ((size_t)d->batch * rows * nsplit * d->heads * d->dim_v * sizeof(uint16_t) + 15) / 16 * 16)
            : nullptr;
    aa.qrows_b = d->n_q;
    aa.B = d->batch;
    aa.rows = rows;
    aa.S = d->n_kv;
    aa.H = d->heads;
    aa.Dk = d->dim_qk;
    aa.Dv = d->dim_v;
    aa.k = d->topk;
    aa.sm_scale = sm_scale;
    e = dsa::launch_sparse_mla(aa, s);
    if (e != hipSuccess) return hip_status(e, "attention launch");
    if (kl) {
      dsa::KlArgs ka{};
      ka.at = aa;
      ka.scores = sc;
      ka.ld = d->n_kv;
      ka.sc_rows_b = L.tc;
      ka.kl = kl + i0;
      e = dsa::launch_indexer_kl(ka, s);
      if (e != hipSuccess) return hip_status(e, "indexer KL launch");
    }
  }
  return ok();
}

// ---- the no-allocation attention call: its split partials live in a
// static device array instead of a caller workspace.  `scratch` names the
// array only in device code; host code uses the address that
// hipGetSymbolAddress returns for the current device (each device holds its
// own copy), taken once per device on the first call there.
constexpr size_t kNoAllocScratchBytes = 40ull << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

struct ScratchAddr {
  std::once_flag flag[dsa::kMaxDevices];
  void* ptr[dsa::kMaxDevices] = {};
  hipError_t err[dsa::kMaxDevices] = {};
};
ScratchAddr g_scratch;

hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= dsa::kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch.flag[dev], [dev] {
    g_scratch.err[dev] = hipGetSymbolAddress(&g_scratch.ptr[dev], HIP_SYMBOL(scratch));
  });
  *out = g_scratch.ptr[dev];
  return g_scratch.err[dev];
}

int kl_impl(const dsa_dims* d, const dsa::PagedKV& pk, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
            const float* lse, const float* scores, int64_t ld, float sm_scale, float* kl, void* stream) {
  int st;
  if ((st = check_common(d)) != DSA_OK) return st;
  if ((st = check_attn_dims(d)) != DSA_OK) return st;
  if (pk.page_table == nullptr && (st = check_dense_kv_size(d)) != DSA_OK) return st;
  REQUIRE(q && kv && idx && lse && scores && kl, DSA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned(q, 16) && aligned(kv, 16) && aligned(idx, 4) && aligned(lse, 4) && aligned(scores, 4) &&
              aligned(kl, 4),
          DSA_ERR_INVALID_ARG, "q and kv must be 16-byte aligned; idx, lse, scores and kl 4-byte aligned");
  REQUIRE(std::isfinite(sm_scale) && sm_scale > 0.f, DSA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  REQUIRE(ld >= d->n_kv, DSA_ERR_INVALID_ARG, "ld (%lld) must be >= n_kv (%d)", (long long)ld, d->n_kv);
  dsa::KlArgs ka{};
  ka.at.pk = pk;
  ka.at.q = q;
  ka.at.kv = kv;
  ka.at.idx = idx;
  ka.at.lse = const_cast<float*>(lse);
  ka.at.qrows_b = d->n_q;
  ka.at.idx_rows_b = d->n_q;
  ka.at.B = d->batch;
  ka.at.rows = d->n_q;
  ka.at.S = d->n_kv;
  ka.at.H = d->heads;
  ka.at.Dk = d->dim_qk;
  ka.at.Dv = d->dim_v;
  ka.at.k = d->topk;
  ka.at.nsplit = 1;
  ka.at.sm_scale = sm_scale;
  ka.scores = scores;
  ka.ld = ld;
  ka.sc_rows_b = d->n_q;
  ka.kl = kl;
  return hip_status(dsa::launch_indexer_kl(ka, (hipStream_t)stream), "indexer KL launch");
}

}  // namespace

extern "C" {

int dsa_indexer_scores(const dsa_dims* d, const uint8_t* q_idx, const float* q_scale, const uint16_t* w_idx,
                       const uint8_t* k_idx, const float* k_scale, float* scores, int64_t ld, void* stream) {
  return indexer_impl(d, dsa::PagedKV{}, q_idx, q_scale, w_idx, k_idx, k_scale, scores, ld, stream);
}

int dsa_topk(const dsa_dims* d, const float* scores, int64_t ld, int32_t* idx, void* stream) {
  return topk_impl(d, dsa::PagedKV{}, scores, ld, idx, stream);
}

size_t dsa_topk_workspace_size(const dsa_dims* d) {
  if (check_common(d) != DSA_OK) return 0;
  return dsa::topk_split_bytes((int64_t)d->batch * d->n_q, topk_call_parts(d));
}

int dsa_topk_ws(const dsa_dims* d, const float* scores, int64_t ld, int32_t* idx, void* ws, size_t ws_bytes,
                void* stream) {
  return topk_impl(d, dsa::PagedKV{}, scores, ld, idx, stream, ws, ws_bytes, true);
}

size_t dsa_attn_workspace_size(const dsa_dims* d) {
  if (check_common(d) != DSA_OK || check_attn_dims(d) != DSA_OK) return 0;
  return attn_partial_bytes(d, d->n_q);
}

int dsa_sparse_mla_attn(const dsa_dims* d, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                        float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return attn_impl(d, dsa::PagedKV{}, q, kv, idx, sm_scale, out, lse, ws, ws_bytes, stream);
}

int dsa_sparse_mla_attn_noalloc(const dsa_dims* d, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                                float sm_scale, uint16_t* out, float* lse, void* stream) {
  int st;
  if ((st = validate_attn(d, q, kv, idx, sm_scale, out, lse, true, true)) != DSA_OK) return st;
  const size_t need = attn_partial_bytes(d, d->n_q);
  REQUIRE(need <= kNoAllocScratchBytes, DSA_ERR_UNSUPPORTED,
          "these dims need %zu bytes of split partials; the no-allocation call holds at most %zu (use "
          "dsa_sparse_mla_attn with a workspace)",
          need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return hip_status(e, "scratch address");
  }
  return attn_impl(d, dsa::PagedKV{}, q, kv, idx, sm_scale, out, lse, ws, need > 0 ? kNoAllocScratchBytes : 0,
                   stream);
}

size_t dsa_forward_workspace_size(const dsa_dims* d) {
  if (check_common(d) != DSA_OK || check_indexer_dims(d) != DSA_OK || check_attn_dims(d) != DSA_OK) return 0;
  return forward_layout(d).total;
}

int dsa_forward_plan_of(const dsa_dims* d, dsa_forward_plan* plan) {
  int st;
  if ((st = check_common(d)) != DSA_OK) return st;
  if ((st = check_indexer_dims(d)) != DSA_OK) return st;
  if ((st = check_attn_dims(d)) != DSA_OK) return st;
  REQUIRE(plan != nullptr, DSA_ERR_INVALID_ARG, "plan is NULL");
  const ForwardLayout L = forward_layout(d);
  plan->chunk_rows = L.tc;
  plan->topk_parts = L.topk_parts;
  plan->attn_splits = L.attn_splits;
  plan->workspace_bytes = L.total;
  return ok();
}

int dsa_forward(const dsa_dims* d, const uint8_t* q_idx, const float* q_scale, const uint16_t* w_idx,
                const uint8_t* k_idx, const float* k_scale, const uint16_t* q, const uint16_t* kv, float sm_scale,
                uint16_t* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(d, dsa::PagedKV{}, q_idx, q_scale, w_idx, k_idx, k_scale, q, kv, sm_scale, out, lse, idx_out,
                      ws, ws_bytes, stream);
}

#define PAGED_PROLOGUE                                  \
  if (d == nullptr) return fail(DSA_ERR_INVALID_ARG, "dims is NULL"); \
  const dsa_dims dd = paged_dims(d);                    \
  dsa::PagedKV pk;                                      \
  {                                                     \
    const int st_ = check_paged(&dd, layout, &pk);      \
    if (st_ != DSA_OK) return st_;                      \
  }

int dsa_indexer_scores_paged(const dsa_dims* d, const dsa_paged_kv* layout, const uint8_t* q_idx,
                             const float* q_scale, const uint16_t* w_idx, const uint8_t* k_idx, const float* k_scale,
                             float* scores, int64_t ld, void* stream) {
  PAGED_PROLOGUE
  return indexer_impl(&dd, pk, q_idx, q_scale, w_idx, k_idx, k_scale, scores, ld, stream);
}

int dsa_topk_paged(const dsa_dims* d, const dsa_paged_kv* layout, const float* scores, int64_t ld, int32_t* idx,
                   void* stream) {
  PAGED_PROLOGUE
  return topk_impl(&dd, pk, scores, ld, idx, stream);
}

int dsa_sparse_mla_attn_paged(const dsa_dims* d, const dsa_paged_kv* layout, const uint16_t* q, const uint16_t* kv,
                              const int32_t* idx, float sm_scale, uint16_t* out, float* lse, void* ws,
                              size_t ws_bytes, void* stream) {
  PAGED_PROLOGUE
  return attn_impl(&dd, pk, q, kv, idx, sm_scale, out, lse, ws, ws_bytes, stream);
}

int dsa_forward_paged(const dsa_dims* d, const dsa_paged_kv* layout, const uint8_t* q_idx, const float* q_scale,
                      const uint16_t* w_idx, const uint8_t* k_idx, const float* k_scale, const uint16_t* q,
                      const uint16_t* kv, float sm_scale, uint16_t* out, float* lse, int32_t* idx_out, void* ws,
                      size_t ws_bytes, void* stream) {
  PAGED_PROLOGUE
  return forward_impl(&dd, pk, q_idx, q_scale, w_idx, k_idx, k_scale, q, kv, sm_scale, out, lse, idx_out, ws,
                      ws_bytes, stream);
}

// Layout-optional calls: a NULL layout means dense caches.
#define LAYOUT_PROLOGUE                                 \
  if (d == nullptr) return fail(DSA_ERR_INVALID_ARG, "dims is NULL"); \
  dsa::PagedKV pk{};                                    \
  dsa_dims dd = *d;                                     \
  if (layout) {                                         \
    dd = paged_dims(d);                                 \
    const int st_ = check_paged(&dd, layout, &pk);      \
    if (st_ != DSA_OK) return st_;                      \
  }

int dsa_indexer_kl(const dsa_dims* d, const dsa_paged_kv* layout, const uint16_t* q, const uint16_t* kv,
                   const int32_t* idx, const float* lse, const float* scores, int64_t ld, float sm_scale, float* kl,
                   void* stream) {
  LAYOUT_PROLOGUE
  return kl_impl(&dd, pk, q, kv, idx, lse, scores, ld, sm_scale, kl, stream);
}

int dsa_forward_kl(const dsa_dims* d, const dsa_paged_kv* layout, const uint8_t* q_idx, const float* q_scale,
                   const uint16_t* w_idx, const uint8_t* k_idx, const float* k_scale, const uint16_t* q,
                   const uint16_t* kv, float sm_scale, uint16_t* out, float* lse, int32_t* idx_out, float* kl,
                   void* ws, size_t ws_bytes, void* stream) {
  LAYOUT_PROLOGUE
  REQUIRE(kl != nullptr && lse != nullptr, DSA_ERR_INVALID_ARG, "kl and lse are required");
  return forward_impl(&dd, pk, q_idx, q_scale, w_idx, k_idx, k_scale, q, kv, sm_scale, out, lse, idx_out, ws,
                      ws_bytes, stream, kl);
}

#undef LAYOUT_PROLOGUE
#undef PAGED_PROLOGUE

int dsa_validate(const dsa_dims* d, const dsa_paged_kv* layout, const float* q_scale, const uint16_t* w_idx,
                 const float* k_scale, const int32_t* idx, int32_t* counts, void* stream) {
  if (d == nullptr) return fail(DSA_ERR_INVALID_ARG, "dims is NULL");
  dsa::PagedKV pk{};
  dsa_dims dd = *d;
  if (layout) {
    dd = paged_dims(d);
    const int st = check_paged(&dd, layout, &pk);
    if (st != DSA_OK) return st;
  }
  int st;
  if ((st = check_common(&dd)) != DSA_OK) return st;
  REQUIRE(counts != nullptr && aligned(counts, 4), DSA_ERR_INVALID_ARG, "counts must be a 4-byte aligned device pointer");
  REQUIRE(aligned(q_scale, 4) && aligned(k_scale, 4) && aligned(idx, 4) && aligned(w_idx, 2), DSA_ERR_INVALID_ARG,
          "misaligned scale/weight/idx pointer");
  REQUIRE(w_idx == nullptr || (dd.idx_heads >= 1 && dd.idx_heads <= 64), DSA_ERR_UNSUPPORTED,
          "idx_heads must be in [1, 64] (got %d)", dd.idx_heads);
  dsa::ValidateArgs a{};
  a.q_scale = q_scale;
  a.w = w_idx;
  a.k_scale = k_scale;
  a.idx = idx;
  a.counts = counts;
  a.B = dd.batch;
  a.n_q = dd.n_q;
  a.S = dd.n_kv;
  a.HI = dd.idx_heads;
  a.k = dd.topk;
  a.q_pos0 = dd.q_pos0;
  a.pk = pk;
  return hip_status(dsa::launch_validate(a, (hipStream_t)stream), "validate launch");
}

int dsa_gather_stats(const dsa_dims* d, int32_t page_size, const int32_t* idx, int32_t* stats, void* stream) {
  REQUIRE(d != nullptr, DSA_ERR_INVALID_ARG, "dims is NULL");
  REQUIRE(d->batch >= 1 && d->n_q >= 1, DSA_ERR_INVALID_ARG, "batch and n_q must be >= 1 (got %d, %d)", d->batch,
          d->n_q);
  REQUIRE((int64_t)d->batch * d->n_q <= (1ll << 30), DSA_ERR_UNSUPPORTED, "batch * n_q too large");
  REQUIRE(d->topk >= 1 && d->topk <= 2048, DSA_ERR_UNSUPPORTED, "topk must be in [1, 2048] (got %d)", d->topk);
  REQUIRE(page_size >= 1, DSA_ERR_INVALID_ARG, "page_size must be >= 1 (got %d)", page_size);
  REQUIRE(idx && stats, DSA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned(idx, 4) && aligned(stats, 4), DSA_ERR_INVALID_ARG, "misaligned idx/stats pointer");
  return hip_status(dsa::launch_gather_stats(idx, stats, (int64_t)d->batch * d->n_q, d->topk, page_size,
                                             (hipStream_t)stream),
                    "gather stats launch");
}

}  // extern "C"

extern "C" {

int dsa_quantize_e4m3(const void* x, int x_dtype, int64_t n_tokens, int32_t token_len, uint8_t* codes,
                      float* scales, void* stream) {
  REQUIRE(x && codes && scales, DSA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(x_dtype == 0 || x_dtype == 1, DSA_ERR_INVALID_ARG, "x_dtype must be 0 (f32) or 1 (bf16), got %d", x_dtype);
  REQUIRE(n_tokens >= 0 && n_tokens <= (1ll << 30), DSA_ERR_INVALID_ARG, "n_tokens out of range (%lld)",
          (long long)n_tokens);
  REQUIRE(token_len >= 4 && token_len <= 16384 && token_len % 4 == 0, DSA_ERR_UNSUPPORTED,
          "token_len must be a multiple of 4 in [4, 16384] (got %d)", token_len);
  REQUIRE(aligned(x, x_dtype == 0 ? 16 : 8) && aligned(codes, 4) && aligned(scales, 4), DSA_ERR_INVALID_ARG,
          "misaligned x/codes/scales pointer");
  return hip_status(dsa::launch_quantize(x, x_dtype, n_tokens, token_len, (int32_t)std::max<int64_t>(n_tokens, 1),
                                         0, 0, codes, scales, (hipStream_t)stream),
                    "quantize launch");
}

int dsa_cache_append(const dsa_dims* d, const void* k_new, int k_dtype, const uint16_t* kv_new, uint8_t* k_idx,
                     float* k_scale, uint16_t* kv, void* stream) {
  REQUIRE(d != nullptr, DSA_ERR_INVALID_ARG, "dims is NULL");
  REQUIRE(d->batch >= 1 && d->n_q >= 1 && d->n_kv >= 1, DSA_ERR_INVALID_ARG,
          "batch, n_q and n_kv must be >= 1 (got %d, %d, %d)", d->batch, d->n_q, d->n_kv);
  REQUIRE(d->q_pos0 >= 0 && (int64_t)d->q_pos0 + d->n_q <= d->n_kv, DSA_ERR_INVALID_ARG,
          "new positions q_pos0 .. q_pos0 + n_q - 1 must lie inside the cache (q_pos0 %d, n_q %d, n_kv %d)",
          d->q_pos0, d->n_q, d->n_kv);
  REQUIRE((int64_t)d->batch * d->n_q <= (1ll << 30), DSA_ERR_UNSUPPORTED, "batch * n_q too large");
  REQUIRE(k_new && k_idx && k_scale, DSA_ERR_INVALID_ARG, "null key pointer");
  REQUIRE(k_dtype == 0 || k_dtype == 1, DSA_ERR_INVALID_ARG, "k_dtype must be 0 (f32) or 1 (bf16), got %d", k_dtype);
  REQUIRE(d->idx_dim >= 4 && d->idx_dim <= 16384 && d->idx_dim % 4 == 0, DSA_ERR_UNSUPPORTED,
          "idx_dim must be a multiple of 4 in [4, 16384] (got %d)", d->idx_dim);
  REQUIRE(aligned(k_new, k_dtype == 0 ? 16 : 8) && aligned(k_idx, 4) && aligned(k_scale, 4), DSA_ERR_INVALID_ARG,
          "misaligned key pointer");
  REQUIRE((kv_new == nullptr) == (kv == nullptr), DSA_ERR_INVALID_ARG, "kv_new and kv must both be given or both NULL");
  if (kv) {
    REQUIRE(d->dim_qk >= 8 && d->dim_qk % 8 == 0, DSA_ERR_UNSUPPORTED, "dim_qk must be a multiple of 8 (got %d)",
            d->dim_qk);
    REQUIRE(aligned(kv_new, 16) && aligned(kv, 16), DSA_ERR_INVALID_ARG, "kv_new and kv must be 16-byte aligned");
  }
  const hipStream_t s = (hipStream_t)stream;
  const int64_t n = (int64_t)d->batch * d->n_q;
  int st = hip_status(dsa::launch_quantize(k_new, k_dtype, n, d->idx_dim, d->n_q, d->n_kv, d->q_pos0, k_idx, k_scale, s),
                      "cache append (keys)");
  if (st != DSA_OK || !kv) return st;
  return hip_status(dsa::launch_copy_rows(kv_new, kv, n, d->dim_qk, d->n_q, d->n_kv, d->q_pos0, s),
                    "cache append (latents)");
}

}  // extern "C"

// ---------------------------------------------------------------- masked MHA mode (short prefill)
namespace {

constexpr int kMhaMaxKv = 65536;   // the selection bitmap of a row is staged whole in LDS

int check_mha(const dsa_dims* d, int dn, int dvh) {
  int st;
  if ((st = check_common(d)) != DSA_OK) return st;
  REQUIRE(d->heads >= 1 && d->heads <= 128, DSA_ERR_UNSUPPORTED, "heads must be in [1, 128] (got %d)", d->heads);
  REQUIRE(d->dim_v >= 1 && d->dim_v < d->dim_qk, DSA_ERR_INVALID_ARG,
          "dim_v (%d) must be below dim_qk (%d): MHA mode needs rope dims", d->dim_v, d->dim_qk);
  REQUIRE(dsa::mha_dims_supported(dn, d->dim_qk - d->dim_v, dvh, d->dim_v), DSA_ERR_UNSUPPORTED,
          "MHA dims (dim_nope %d, rope %d, dim_vh %d, dim_v %d) not built; supported: 128/64/128 and 32/16/32 "
          "with dim_v a multiple of 64",
          dn, d->dim_qk - d->dim_v, dvh, d->dim_v);
  REQUIRE(d->n_kv <= kMhaMaxKv, DSA_ERR_UNSUPPORTED, "masked MHA mode supports n_kv <= %d (got %d)", kMhaMaxKv,
          d->n_kv);
  return DSA_OK;
}

int mha_nc(const dsa_dims* d) { return (d->n_kv + 31) / 32; }

int mask_impl(const dsa_dims* d, const int32_t* idx, int64_t idx_rows_b, int rows, int row0, uint32_t* mask,
              hipStream_t s) {
  dsa::MaskArgs m{};
  m.idx = idx;
  m.mask = mask;
  m.idx_rows_b = idx_rows_b;
  m.B = d->batch;
  m.rows = rows;
  m.row0 = row0;
  m.T = d->n_q;
  m.S = d->n_kv;
  m.k = d->topk;
  m.pos0 = d->q_pos0;
  m.NC = mha_nc(d);
  return hip_status(dsa::launch_selection_mask(m, s), "selection mask launch");
}

int decompress_impl(const dsa_dims* d, int dn, int dvh, const uint16_t* kv, const uint16_t* w_uk,
                    const uint16_t* w_uv, int n_rows, int S_h, uint16_t* k_mha, uint16_t* v_mha, hipStream_t s) {
  dsa::DecompArgs a{};
  a.kv = kv;
  a.w[0] = w_uk;
  a.w[1] = w_uv;
  a.out[0] = k_mha;
  a.out[1] = v_mha;
  a.rows_w[0] = dn;
  a.rows_w[1] = dvh;
  a.B = d->batch;
  a.S = d->n_kv;
  a.H = d->heads;
  a.Dk = d->dim_qk;
  a.Dv = d->dim_v;
  a.n_rows = n_rows;
  a.S_h = S_h;
  return hip_status(dsa::launch_mha_decompress(a, s), "MHA decompression launch");
}

int mha_attn_launch(const dsa_dims* d, int dn, int dvh, const uint16_t* q_mha, const uint16_t* kv,
                    const uint16_t* k_mha, const uint16_t* v_mha, int S_h, const uint32_t* mask, float sm_scale,
                    uint16_t* out, float* lse, hipStream_t s) {
  dsa::MhaArgs a{};
  a.q = q_mha;
  a.kv = kv;
  a.kh = k_mha;
  a.vh = v_mha;
  a.mask = mask;
  a.out = out;
  a.lse = lse;
  a.B = d->batch;
  a.T = d->n_q;
  a.S = d->n_kv;
  a.S_h = S_h;
  a.H = d->heads;
  a.Dk = d->dim_qk;
  a.Dv = d->dim_v;
  a.pos0 = d->q_pos0;
  a.NC = mha_nc(d);
  a.sm_scale = sm_scale;
  return hip_status(dsa::launch_masked_mha(a, dn, d->dim_qk - d->dim_v, dvh, s), "masked MHA launch");
}

struct MhaLayout {
  int64_t tc;
  size_t scores_off, idx_off, mask_off, k_off, v_off, total;
};

MhaLayout mha_layout(const dsa_dims* d, int dn, int dvh) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  MhaLayout L;
  L.tc = forward_chunk_rows(d);
  const size_t rows_h = (size_t)d->q_pos0 + d->n_q;   // keys any row can see
  L.scores_off = 0;
  L.idx_off = up((size_t)d->batch * L.tc * d->n_kv * sizeof(float));
  L.mask_off = L.idx_off + up((size_t)d->batch * L.tc * d->topk * sizeof(int32_t));
  L.k_off = L.mask_off + up((size_t)d->batch * mha_nc(d) * d->n_q * sizeof(uint32_t));
  L.v_off = L.k_off + up((size_t)d->batch * d->heads * rows_h * dn * 2);
  L.total = L.v_off + up((size_t)d->batch * d->heads * rows_h * dvh * 2);
  return L;
}

}  // namespace

extern "C" {

int dsa_selection_mask(const dsa_dims* d, const int32_t* idx, uint32_t* mask, void* stream) {
  int st;
  if ((st = check_common(d)) != DSA_OK) return st;
  REQUIRE(d->n_kv <= kMhaMaxKv, DSA_ERR_UNSUPPORTED, "selection masks support n_kv <= %d (got %d)", kMhaMaxKv,
          d->n_kv);
  REQUIRE(idx && mask, DSA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned(idx, 4) && aligned(mask, 4), DSA_ERR_INVALID_ARG, "idx and mask must be 4-byte aligned");
  return mask_impl(d, idx, d->n_q, d->n_q, 0, mask, (hipStream_t)stream);
}

int dsa_mha_decompress(const dsa_dims* d, int32_t dim_nope, int32_t dim_vh, const uint16_t* kv, const uint16_t* w_uk,
                       const uint16_t* w_uv, int32_t n_rows, uint16_t* k_mha, uint16_t* v_mha, void* stream) {
  int st;
  if ((st = check_mha(d, dim_nope, dim_vh)) != DSA_OK) return st;
  REQUIRE(kv && w_uk && w_uv && k_mha && v_mha, DSA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned(kv, 16) && aligned(w_uk, 16) && aligned(w_uv, 16) && aligned(k_mha, 16) && aligned(v_mha, 16),
          DSA_ERR_INVALID_ARG, "kv, w_uk, w_uv, k_mha and v_mha must be 16-byte aligned");
  REQUIRE(n_rows >= 0 && n_rows <= d->n_kv, DSA_ERR_INVALID_ARG, "n_rows (%d) must be in [0, n_kv = %d]", n_rows,
          d->n_kv);
  return decompress_impl(d, dim_nope, dim_vh, kv, w_uk, w_uv, n_rows, d->n_kv, k_mha, v_mha, (hipStream_t)stream);
}

int dsa_masked_mha_attn(const dsa_dims* d, int32_t dim_nope, int32_t dim_vh, const uint16_t* q_mha,
                        const uint16_t* kv, const uint16_t* k_mha, const uint16_t* v_mha, const uint32_t* mask,
                        float sm_scale, uint16_t* out, float* lse, void* stream) {
  int st;
  if ((st = check_mha(d, dim_nope, dim_vh)) != DSA_OK) return st;
  REQUIRE(q_mha && kv && k_mha && v_mha && mask && out, DSA_ERR_INVALID_ARG, "null tensor pointer");
  REQUIRE(aligned(q_mha, 16) && aligned(kv, 16) && aligned(k_mha, 16) && aligned(v_mha, 16) && aligned(out, 16) &&
              aligned(mask, 4) && aligned(lse, 4),
          DSA_ERR_INVALID_ARG, "q_mha, kv, k_mha, v_mha and out must be 16-byte aligned; mask and lse 4-byte aligned");
  REQUIRE(std::isfinite(sm_scale) && sm_scale > 0.f, DSA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  return mha_attn_launch(d, dim_nope, dim_vh, q_mha, kv, k_mha, v_mha, d->n_kv, mask, sm_scale, out, lse,
                         (hipStream_t)stream);
}

size_t dsa_masked_mha_workspace_size(const dsa_dims* d, int32_t dim_nope, int32_t dim_vh) {
  if (check_mha(d, dim_nope, dim_vh) != DSA_OK || check_indexer_dims(d) != DSA_OK) return 0;
  return mha_layout(d, dim_nope, dim_vh).total;
}

int dsa_masked_mha_forward(const dsa_dims* d, int32_t dim_nope, int32_t dim_vh, const uint8_t* q_idx,
                           const float* q_scale, const uint16_t* w_idx, const uint8_t* k_idx, const float* k_scale,
                           const uint16_t* q_mha, const uint16_t* kv, const uint16_t* w_uk, const uint16_t* w_uv,
                           float sm_scale, uint16_t* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                           void* stream) {
  int st;
  if ((st = check_mha(d, dim_nope, dim_vh)) != DSA_OK) return st;
  if ((st = check_indexer_dims(d)) != DSA_OK) return st;
  REQUIRE(q_idx && q_scale && w_idx && k_idx && k_scale && q_mha && kv && w_uk && w_uv && out, DSA_ERR_INVALID_ARG,
          "null tensor pointer");
  REQUIRE(aligned(q_idx, 16) && aligned(k_idx, 16), DSA_ERR_INVALID_ARG, "q_idx and k_idx must be 16-byte aligned");
  REQUIRE(aligned(q_scale, 4) && aligned(k_scale, 4) && aligned(w_idx, 2) && aligned(idx_out, 4) && aligned(lse, 4),
          DSA_ERR_INVALID_ARG, "misaligned scale/weight/idx/lse pointer");
  REQUIRE(aligned(q_mha, 16) && aligned(kv, 16) && aligned(w_uk, 16) && aligned(w_uv, 16) && aligned(out, 16),
          DSA_ERR_INVALID_ARG, "q_mha, kv, w_uk, w_uv and out must be 16-byte aligned");
  REQUIRE(std::isfinite(sm_scale) && sm_scale > 0.f, DSA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const MhaLayout L = mha_layout(d, dim_nope, dim_vh);
  REQUIRE(ws != nullptr && ws_bytes >= L.total, DSA_ERR_WORKSPACE,
          "masked MHA forward needs %zu workspace bytes (got %zu)", L.total, ws ? ws_bytes : (size_t)0);
  REQUIRE(aligned(ws, 256), DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");

  const hipStream_t s = (hipStream_t)stream;
  char* wsb = (char*)ws;
  float* sc = (float*)(wsb + L.scores_off);
  uint32_t* mask = (uint32_t*)(wsb + L.mask_off);
  uint16_t* k_mha = (uint16_t*)(wsb + L.k_off);
  uint16_t* v_mha = (uint16_t*)(wsb + L.v_off);
  const bool decode_form = d->n_q <= dsa::kIndexerDecodeMaxRows;
  for (int64_t i0 = 0; i0 < d->n_q; i0 += L.tc) {
    const int rows = (int)((d->n_q - i0) < L.tc ? (d->n_q - i0) : L.tc);
    const dsa::IndexerArgs ia =
        indexer_args(d, q_idx, q_scale, w_idx, k_idx, k_scale, sc, d->n_kv, i0, rows, L.tc, dsa::PagedKV{});
    hipError_t e = dsa::launch_indexer(ia, decode_form, s);
    if (e != hipSuccess) return hip_status(e, "indexer launch");
    dsa::TopkArgs ta{};
    ta.scores = sc;
    ta.ld = d->n_kv;
    ta.sc_rows_b = L.tc;
    ta.idx = idx_out ? idx_out + i0 * d->topk : (int32_t*)(wsb + L.idx_off);
    ta.idx_rows_b = idx_out ? d->n_q : L.tc;
    ta.B = d->batch;
    ta.rows = rows;
    ta.pos0 = d->q_pos0 + (int)i0;
    ta.S = d->n_kv;
    ta.k = d->topk;
    e = dsa::launch_topk(ta, s);
    if (e != hipSuccess) return hip_status(e, "top-k launch");
    if ((st = mask_impl(d, ta.idx, ta.idx_rows_b, rows, (int)i0, mask, s)) != DSA_OK) return st;
  }
  const int rows_h = d->q_pos0 + d->n_q;
  if ((st = decompress_impl(d, dim_nope, dim_vh, kv, w_uk, w_uv, rows_h, rows_h, k_mha, v_mha, s)) != DSA_OK)
    return st;
  return mha_attn_launch(d, dim_nope, dim_vh, q_mha, kv, k_mha, v_mha, rows_h, mask, sm_scale, out, lse, s);
}

}  // extern "C"
