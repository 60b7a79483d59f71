// Internal launch interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// A span of query rows: rows [0, rows) of each of B sequences, where row i
// sits at absolute position pos0 + i.  Row-indexed tensors advance by
// `qrows_b` rows from one sequence to the next.
struct IndexerArgs {
  const uint8_t* q_idx;   // [B, qrows_b, HI, dI] e4m3
  const float* q_scale;   // [B, qrows_b]
  const uint16_t* w;      // [B, qrows_b, HI] bf16
  const uint8_t* k_idx;   // [B, S, dI] e4m3
  const float* k_scale;   // [B, S]
  float* scores;          // [B, sc_rows_b, ld]
  int64_t ld;
  int64_t qrows_b;
  int64_t sc_rows_b;
  int B, rows, pos0, S, HI, dI;
};

struct TopkArgs {
  const float* scores;    // [B, sc_rows_b, ld]
  int32_t* idx;           // [B, idx_rows_b, k]
  int64_t ld;
  int64_t sc_rows_b;
  int64_t idx_rows_b;
  int B, rows, pos0, S, k;
};

struct AttnArgs {
  const uint16_t* q;      // [B, qrows_b, H, Dk] bf16
  const uint16_t* kv;     // [B, S, Dk] bf16
  const int32_t* idx;     // [B, idx_rows_b, k]
  uint16_t* out;          // [B, qrows_b, H, Dv] bf16
  float* lse;             // [B, qrows_b, H] or null
  float* part_o;          // split partials [B*rows, nsplit, H, Dv] f32 (nsplit > 1)
  float* part_lse;        // [B*rows, nsplit, H]
  int64_t qrows_b;        // row stride between sequences for q, out, lse
  int64_t idx_rows_b;     // row stride between sequences for idx
  int B, rows, S, H, Dk, Dv, k, nsplit;
  float sm_scale;
};

// Kernel choice for the indexer: decode form (one row per wave, keys split
// across waves) for spans of at most this many rows per sequence.
constexpr int kIndexerDecodeMaxRows = 4;

hipError_t launch_indexer(const IndexerArgs& a, bool decode_form, hipStream_t st);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
hipError_t launch_sparse_mla(const AttnArgs& a, hipStream_t st);

// Shape support checks (true if the kernels are built for these dims).
bool attn_dims_supported(int H, int Dk, int Dv);
int topk_max_kv();

// Per-token E4M3 quantisation of n_tokens rows of len values (dtype 0 f32,
// 1 bf16); token tok goes to output row (tok / group) * out_stride + out_off
// + tok % group of codes/scales.
hipError_t launch_quantize(const void* x, int dtype, int64_t n_tokens, int32_t len, int32_t group,
                           int64_t out_stride, int64_t out_off, uint8_t* codes, float* scales, hipStream_t st);
// Copy of n_rows bf16 rows of row_len (a multiple of 8) with the same row mapping.
hipError_t launch_copy_rows(const uint16_t* src, uint16_t* dst, int64_t n_rows, int32_t row_len, int32_t group,
                            int64_t out_stride, int64_t out_off, hipStream_t st);

}  // namespace dsa
