// Internal declarations shared by the host entry points and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Arguments of the fused ring + current attention kernel.  All sizes are
// validated by the host before launch; 32-bit byte offsets are proven to fit.
struct FusedParams {
  const uint16_t* q;        // bf16 [C, NQ, HD]
  const uint16_t* k_cache;  // bf16 [P, shard_cap, NKV, HD]
  const uint16_t* v_cache;
  const uint16_t* k_cur;    // bf16 [cur_len, NKV, HD], token order
  const uint16_t* v_cur;
  void* out;                // [C, NQ, HD] bf16 | fp32
  float* lse;               // [NQ, C] or nullptr
  int64_t shard_cap;        // slots per shard
  int64_t full;             // cache_len / (P * I)
  int64_t rem;              // cache_len % (P * I)
  int32_t P, interleave, ring_start;
  int32_t nb;               // ring tiles per shard visit (max shard length / BKV, rounded up)
  int32_t nq, nkv, group;   // group = NQ / NKV
  int32_t q_rows, real_rows;
  int32_t head_rows;        // rows of the head piece; the rest is the tail piece
  int32_t head_pos, tail_pos;  // chunk positions of the first head / tail row
  int32_t row_tiles;        // row tiles per KV head
  int32_t splits;           // segments the tile walk of a row tile is cut into
  int32_t seg_tiles;        // tiles per segment (the last one of a row tile may be shorter)
  int64_t seg_out_stride;   // elements between the segments' partial outputs
  int32_t grid_real;        // row_tiles * splits * NKV
  int32_t out_f32;          // fp32 output numerics: exact running max, sums of rounded probabilities
  int32_t store_f32;        // out is written in fp32 (out_f32, or a split launch's partials)
  int32_t regions;          // 1: cache (ring) only, 2: current only, 3: both
  float scale_log2e;        // softmax scale * log2(e)
  // The strided cache write fused into the launch (write_tokens > 0): current
  // token t < write_tokens goes to global position write_pos0 + t of
  // wk_cache / wv_cache, each workgroup copying write_per_wg tokens.
  uint16_t* wk_cache;
  uint16_t* wv_cache;
  int64_t write_pos0;
  int32_t write_tokens;
  int32_t write_per_wg;
  int32_t write_chunks;     // 16-byte chunks per token row (NKV * HD / 8)
};

// Arguments of the log-sum-exp merge of two partial attentions.
struct MergeParams {
  const void* o1;           // [C, NQ, HD] bf16 | fp32 (parts_f32)
  const float* lse1;        // fp32 [NQ, C]
  const void* o2;
  const float* lse2;
  void* out;                // [C, NQ, HD] bf16 | fp32
  float* lse;               // [NQ, C] or nullptr
  int32_t q_rows, real_rows, nq, hd;
  int32_t parts_f32, out_f32;
};

struct WriteParams {
  const uint16_t* k_cur;
  const uint16_t* v_cur;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int64_t cache_len;
  int64_t shard_cap;
  int32_t n_tokens, P, interleave;
  int32_t row_chunks;       // 16-byte chunks per token row (NKV * HD / 8)
};

// Tile geometry of the fused kernel for a head dimension.
constexpr int kWaves = 4;           // waves per workgroup
constexpr int kRowsPerWave = 64;    // (token, head) rows per wave (two 32-row MFMA blocks)
constexpr int kRowsPerWG = kWaves * kRowsPerWave;
constexpr int kBKV = 32;            // keys per KV tile
// Workgroups of the fused kernel resident per CU: two at HD = 64 (32 KiB
// of LDS and 256 registers per lane each), one otherwise.
template <int D>
constexpr int kWGsPerCU = D == 64 ? 2 : 1;
constexpr int wgs_per_cu(int head_dim) { return head_dim == 64 ? 2 : 1; }

hipError_t launch_fused(const FusedParams& p, int head_dim, hipStream_t stream);
hipError_t launch_kv_cache_write(const WriteParams& p, hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);

// Arguments of the S-way merge of a split launch's partials.
struct MergeSplitsParams {
  const void* part_o;       // [S, C, NQ, HD] bf16 | fp32 (parts_f32)
  const float* part_lse;    // [S, NQ, C]
  void* out;                // [C, NQ, HD] bf16 | fp32
  float* lse;               // [NQ, C] or nullptr
  int32_t splits, q_rows, real_rows, nq, hd;
  int32_t parts_f32, out_f32;
};
hipError_t launch_merge_splits(const MergeSplitsParams& p, hipStream_t stream);

}  // namespace ra
