// Fused ring + current causal attention for gfx950 (MI355X).
//
// Method: vLLM tpu-inference pull request "PCP: in-kernel ring cache phase,
// fused with the current phase".  Summary: ring cache rounds and the causal
// current phase in one launch sharing one online softmax, no LSE merge.
// Design: per query block, a virtual key-tile index walks the ring region
// (each striped shard in turn) and then the current-KV tiles; region
// behaviour is chosen by value (fetch sizes, one mask bound), not by
// separate code paths.
//
// Mapping onto CDNA4:
//  * A workgroup owns 128 (token, query-head) rows of ONE KV head: the GQA
//    group's query heads are packed into the rows, so every K/V tile is
//    fetched once per group.  Each of the 4 waves owns 32 rows and keeps its
//    Q rows in registers for the whole walk.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then holds 16 keys of ONE row, so
//    the row max / sum are in-lane plus one exchange with lane^32, and the
//    probabilities are already laid out as the B operand of O^T = V^T P^T
//    (the key order inside a 16-key step is permuted identically on both
//    operands, which leaves the contraction unchanged).
//  * K/V tiles are staged in LDS, double buffered (the two "bkv slots"),
//    row-major with a 16-byte-chunk XOR swizzle.  V^T operands are read with
//    ds_read_b64_tr_b16, which transposes 4x16 blocks in flight.
//  * Fetches go through buffer descriptors whose size is the valid length of
//    the visited region: rows past a shard's length (or past the real chunk
//    rows) come back as zeros without touching memory -- the zero-size fetch
//    of the inactive region, chosen by value.  The mask is one bound per
//    lane, key < lim, with lim = shard length in the ring region and
//    token + 1 (causal) in the current region.
//  * Workgroup ids are remapped so that the workgroups resident on one XCD
//    share a KV head and walk the same tiles, keeping the re-streamed K/V in
//    that XCD's L2.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

// XOR pattern for the 16-byte chunk index of LDS tile row `row`.  For a
// 512-byte row it makes both access patterns conflict-free: 16 consecutive
// rows at one chunk (K operand reads) and 4 consecutive rows x 4 chunks
// (transposed V reads).
__device__ __forceinline__ int swz(int row, int cpr) {
  return (4 * (row & 3) + ((row >> 2) & 3)) & (cpr - 1);
}

// Element offset of (row, col) in an LDS tile stored [rows][D], swizzled.
template <int D>
__device__ __forceinline__ int lds_off(int row, int col) {
  return row * D + (((col >> 3) ^ swz(row, D / 8)) << 3) + (col & 7);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer (stride 0): loads at byte offsets >= `bytes` return zero.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void ring_attn_fused_kernel(FusedParams p) {
  constexpr int NT = kWaves * 64;
  constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  constexpr int NKB = kBKV / 32;          // 32-key blocks per tile
  constexpr int NDB = D / 32;             // 32-wide d blocks of the output
  constexpr int NKS = D / 16;             // k-steps of the QK^T contraction
  constexpr int TILE = kBKV * D;          // elements of one K or V tile
  constexpr int LOADS = kBKV * CPR / NT;  // 16-byte chunks per thread per tile
  static_assert((kBKV * CPR) % NT == 0, "tile must split evenly over threads");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * TILE];  // [slot][K, V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;   // lane half: keys / d interleave of the MFMA layouts
  const int lr = lane & 31;  // row within the wave

  // XCD-aware workgroup order (grid is a multiple of 8).
  const int nwg = gridDim.x;
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nwg >> 3) + (bid >> 3);
  if (logical >= p.grid_real) return;
  const int g = logical / p.row_tiles;
  const int rt = p.row_tiles - 1 - (logical - g * p.row_tiles);  // long causal rows first
  const int row0 = rt * kRowsPerWG;

  const int row = row0 + wave * kRowsPerWave + lr;
  const int token = row / p.group;
  const int head = g * p.group + (row - token * p.group);
  const bool row_ok = token < p.real_rows;

  // Q^T operand: lane holds d = 16 s + 8 h + [0, 8) of its row.
  bf16x8 qreg[NKS];
  {
    const uint16_t* qp = p.q + ((int64_t)token * p.nq + head) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      i16x8 x = row_ok ? *reinterpret_cast<const i16x8*>(qp + 16 * s) : i16x8{0, 0, 0, 0, 0, 0, 0, 0};
      qreg[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Tile schedule: ring region = P shard visits of nb tiles, then the
  // current tiles up to this workgroup's last real token.
  const int wg_last = min(p.real_rows - 1, (row0 + kRowsPerWG - 1) / p.group);
  const int n_ring = p.P * p.nb;
  const int n_cur = (wg_last + kBKV) / kBKV;
  const int T = n_ring + n_cur;
  const uint32_t rowstride = (uint32_t)p.nkv * D * 2;  // bytes between tokens
  const uint32_t cur_bytes = (uint32_t)p.real_rows * rowstride;

  // Per-tile source, chosen by value: descriptor, first byte offset and the
  // key bound (relative to the tile) of the ring or the current region.
  struct Src {
    __amdgpu_buffer_rsrc_t kr, vr;
    uint32_t off;
    int lim_uniform;  // ring: valid keys left in the shard
    bool in_ring;
    int tile_key0;    // current: first key position of the tile
  };
  auto source = [&](int v) {
    Src s;
    s.in_ring = v < n_ring;
    if (s.in_ring) {
      const int k = v / p.nb;
      const int b = v - k * p.nb;
      int sh = p.ring_start - k;
      sh += (sh < 0) ? p.P : 0;
      const int64_t len = p.full * p.interleave +
                          min(max(p.rem - (int64_t)sh * p.interleave, (int64_t)0),
                              (int64_t)p.interleave);
      const int64_t base = ((int64_t)sh * p.shard_cap * p.nkv + g) * D;
      const uint32_t bytes = (uint32_t)len * rowstride;
      s.kr = make_rsrc(p.k_cache + base, bytes);
      s.vr = make_rsrc(p.v_cache + base, bytes);
      s.off = (uint32_t)b * kBKV * rowstride;
      s.lim_uniform = (int)(len - (int64_t)b * kBKV);
      s.tile_key0 = 0;
    } else {
      const int c = v - n_ring;
      s.kr = make_rsrc(p.k_cur + g * D, cur_bytes);
      s.vr = make_rsrc(p.v_cur + g * D, cur_bytes);
      s.off = (uint32_t)c * kBKV * rowstride;
      s.lim_uniform = 0;
      s.tile_key0 = c * kBKV;
    }
    return s;
  };

  i32x4 kst[LOADS], vst[LOADS];
  auto load_tile = [&](int v) {
    const Src s = source(v);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = tid + i * NT;
      const int j = q / CPR, c = q % CPR;
      const uint32_t off = s.off + (uint32_t)j * rowstride + c * 16;
      kst[i] = __builtin_amdgcn_raw_buffer_load_b128(s.kr, off, 0, 0);
      vst[i] = __builtin_amdgcn_raw_buffer_load_b128(s.vr, off, 0, 0);
    }
  };
  auto store_tile = [&](int slot) {
    uint16_t* kl = lds + slot * 2 * TILE;
    uint16_t* vl = kl + TILE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int q = tid + i * NT;
      const int j = q / CPR, c = q % CPR;
      const int o = j * D + ((c ^ swz(j, CPR)) << 3);
      *reinterpret_cast<i32x4*>(kl + o) = kst[i];
      *reinterpret_cast<i32x4*>(vl + o) = vst[i];
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;  // running max, log2 units
  float l_run = 0.f;      // running sum over this lane's half of the keys

  if (T > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  // Lane geometry of the transposed V reads (4 x 16 blocks per 16 lanes).
  const int b4 = lane >> 4, i16 = lane & 15;
  const int vcol = 16 * (b4 & 1) + 4 * (i16 & 3);
  const int vrow = 4 * h + (i16 >> 2);

  for (int v = 0; v < T; ++v) {
    if (v + 1 < T) load_tile(v + 1);
    const uint16_t* kl = lds + (v & 1) * 2 * TILE;
    const uint16_t* vl = kl + TILE;
    const Src src = source(v);
    const int lim = src.in_ring ? src.lim_uniform : token + 1 - src.tile_key0;

    // S^T = K Q^T for the tile's 32-key blocks.
    f32x16 S[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      S[kb] = f32x16{};
      const int krow = kb * 32 + lr;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            kl + krow * D + (((2 * s + h) ^ swz(krow, CPR)) << 3));
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[s], S[kb], 0, 0, 0);
      }
    }

    // Online softmax, shared by both regions.  Register i of block kb holds
    // key kb*32 + (i/4)*8 + 4h + i%4 of this lane's row.
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + (i >> 2) * 8 + 4 * h + (i & 3);
        float t = S[kb][i] * p.scale_log2e;
        t = key < lim ? t : kNegInf;
        S[kb][i] = t;
        mx = fmaxf(mx, t);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float ls = 0.f;
    bf16x8 pb[2 * NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(S[kb][i] - m_use);
        ls += e;
        pb[2 * kb + (i >> 3)][i & 7] = (__bf16)e;
      }
    }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;

    // O^T += V^T P^T, 16 keys per step.
#pragma unroll
    for (int ks = 0; ks < kBKV / 16; ++ks) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int r = 16 * ks + vrow;
        const int col = db * 32 + vcol;
        const i16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vl + lds_off<D>(r, col)));
        const i16x4 x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(vl + lds_off<D>(r + 8, col)));
        const i16x8 x = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), pb[ks],
                                                          acc[db], 0, 0, 0);
      }
    }

    if (v + 1 < T) store_tile((v + 1) & 1);
    __syncthreads();
  }

  // Epilogue: out = acc / l, lse = ln 2 * (m + log2 l).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_ok) {
    const float inv = 1.f / l_tot;
    const int64_t obase = ((int64_t)token * p.nq + head) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = db * 32 + i4 * 8 + 4 * h;
        const f32x4 o = {acc[db][4 * i4] * inv, acc[db][4 * i4 + 1] * inv,
                         acc[db][4 * i4 + 2] * inv, acc[db][4 * i4 + 3] * inv};
        if (p.out_f32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + obase + d0) = o;
        } else {
          typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
          const bf16x4 ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
          *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.out) + obase + d0) = ob;
        }
      }
    }
    if (h == 0 && p.lse != nullptr)
      p.lse[(int64_t)head * p.q_rows + token] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace

hipError_t launch_fused(const FusedParams& p, int head_dim, hipStream_t stream) {
  const int grid = (p.grid_real + 7) / 8 * 8;
  const dim3 block(kWaves * 64);
  switch (head_dim) {
    case 64:
      hipLaunchKernelGGL(ring_attn_fused_kernel<64>, dim3(grid), block, 0, stream, p);
      break;
    case 128:
      hipLaunchKernelGGL(ring_attn_fused_kernel<128>, dim3(grid), block, 0, stream, p);
      break;
    case 256:
      hipLaunchKernelGGL(ring_attn_fused_kernel<256>, dim3(grid), block, 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
