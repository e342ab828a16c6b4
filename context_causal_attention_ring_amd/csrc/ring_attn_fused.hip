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
//  * A workgroup owns 256 (token, query-head) rows of ONE KV head: the GQA
//    group's query heads are packed into the rows, so every K/V tile is
//    fetched once per group.  Each of the 4 waves (one per SIMD) owns 64
//    rows as two 32-row blocks and keeps their Q in registers for the whole
//    walk; every K or V operand read from LDS feeds two MFMAs.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: each lane then holds 16 keys of ONE row, so
//    the row max / sum are in-lane plus one exchange with lane^32, and the
//    probabilities are already laid out as the B operand of O^T = V^T P^T
//    (the key order inside a 16-key step is permuted identically on both
//    operands, which leaves the contraction unchanged).  The fp32
//    accumulator (64 rows x HD) lives in the AGPRs; at HD = 256 the score
//    MFMAs are one asm block that writes the scores to VGPRs, where the
//    softmax reads them.
//  * K/V tiles of 32 keys go HBM -> LDS by buffer_load ... lds (no register
//    staging) into two K and two V slots: while tile v's scores are
//    computed, K of tile v+1 and V of tile v are in flight and the values of
//    tile v-1 are still being consumed.
//    Rows are stored with a 16-byte-chunk XOR swizzle chosen per operand so
//    that K reads (32 rows, one chunk) and transposed V reads
//    (ds_read_b64_tr_b16, 4 rows x 4 chunks) are both bank-conflict free.
//  * Fetches go through buffer descriptors whose size is the valid length
//    of the visited region: rows past a shard's length (or past the real
//    chunk rows) come back as zeros without touching memory -- the
//    zero-size fetch of the inactive region, chosen by value.  The mask is
//    one bound per row, key < lim, with lim = shard length in the ring
//    region and token + 1 (causal) in the current region; tiles that no
//    bound cuts skip the compare entirely.
//  * Online softmax in log2 units with a lazy running max: the
//    accumulator is rescaled only when some row's max grows by more than
//    kTau (a wave vote), so the common tile costs max, fma, exp2, add and
//    a bf16 pack per score.  The softmax of tile v is issued between the
//    P.V MFMAs of tile v-1, which do not depend on it, in a hand-ordered
//    block (one MFMA pair, one V operand read, a slice of softmax work).
//  * Workgroup ids are remapped so that the workgroups resident on one XCD
//    share a KV head and walk the same tiles, keeping the re-streamed K/V in
//    that XCD's L2.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
// Lazy-rescale threshold (log2 units): probabilities stay <= 2^kTau.  With
// fp32 output the running max is exact (threshold 0), so the dominant
// probability of each row is exactly 1 and carries no bf16 rounding.
template <bool F32OUT>
constexpr float kTau = F32OUT ? 0.0f : 8.0f;

// Chunk swizzles (16-byte chunks within a tile row).  K rows are read 32 at
// a time at one chunk: 16 consecutive rows must land in 16 distinct bank
// groups.  V rows are read by the transposing loads as 4 rows x 4 chunks:
// 4*(row & 3) spreads them, and rows r and r + 8 (the two reads of one
// operand) share a pattern so their addresses differ by a constant.
__device__ __forceinline__ int swz_k(int row, int cpr) {
  return (4 * (row & 3) + ((row >> 2) & 3)) & (cpr - 1);
}
__device__ __forceinline__ int swz_v(int row, int cpr) { return (4 * (row & 3)) & (cpr - 1); }

// The same descriptor as four dwords (for the inline-asm LDS copies):
// base address, stride 0, size in bytes, raw-buffer format word.
__device__ __forceinline__ i32x4 make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer (stride 0): loads at byte offsets >= `bytes` return zero.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 bytes per lane from a buffer into LDS at dst + 16 * lane
// (buffer_load_dwordx4 ... lds; M0 holds the LDS address).  Issued through
// inline asm so that the compiler does not make every later LDS read wait
// for it: the kernel orders these copies itself (s_waitcnt vmcnt(0) and a
// barrier before a slot is read, and a barrier after its last read before
// it is refilled).
__device__ __forceinline__ void dma16(const i32x4& rs, uint16_t* dst, uint32_t voff,
                                      uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  // the low 32 bits of a generic LDS address are the LDS offset
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(m0), "v"(voff), "s"(rs), "s"(soff)
      : "memory", "m0");
#endif
}

__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t* base, uint32_t byte_off) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(base) + byte_off);
}

__device__ __forceinline__ i16x4 lds_read_tr(const uint16_t* base, uint32_t byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(reinterpret_cast<const char*>(base) + byte_off));
}

// acc *= alpha on a 16-wide accumulator kept in AGPRs: read, multiply and
// write back in place, so the accumulator never needs a VGPR home.  The
// caller waits out the MFMA result hazard (see rescale_agprs).
__device__ __forceinline__ void scale_agprs(f32x16& a, float alpha) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only parses device code
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = a[i];
    float t;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(t)
        : "v"(alpha));
    a[i] = x;
  }
#endif
}

__device__ __forceinline__ float wave_max_pair(float x) {
  // max with the lane 32 apart (the other half of the same row's keys):
  // v_permlane32_swap exchanges the two lane halves, and the max over
  // {own, both swap results} holds the partner's value in every lane.
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_elementwise_maximum(
      __builtin_elementwise_maximum(x, __uint_as_float(r[0])), __uint_as_float(r[1]));
}

// S^T = K Q^T of one 32-key tile for two 32-row blocks at HD = 256, as one
// asm block so that the scores land in VGPRs (the softmax reads them with
// VALU instructions).  With every MFMA in AGPR form the compiler would
// produce the scores in AGPRs and copy them out, and at this register
// pressure it also copies Q operands around and spills.
//   ka[j]  LDS byte address of this lane's K row at chunk (2j + h) ^ swizzle;
//          k-step s reads ka[s % 8] + 256 (s / 8)
//   q      the Q^T operands of the two row blocks, 16 k-steps each
// K operands are read two k-steps ahead into a ring of three registers;
// LDS reads complete in order, so lgkmcnt(2) before step s means the read
// of step s has landed.  The leading s_nop covers a VALU write of an
// operand just before the first MFMA reads it; the trailing ones cover the
// last MFMA's result before VALU instructions read the scores.
#define RA_KREAD(t, a, off) "ds_read_b128 %[" #t "], %[" #a "] offset:" #off "\n\t"
#define RA_QK2(t, step, c0, c1)                                              \
  "v_mfma_f32_32x32x16_bf16 %[s0], %[" #t "], %[q0_" #step "], " c0 "\n\t" \
  "v_mfma_f32_32x32x16_bf16 %[s1], %[" #t "], %[q1_" #step "], " c1 "\n\t"
#define RA_QK(t, step) RA_QK2(t, step, "%[s0]", "%[s1]")
#define RA_WAIT(n) "s_waitcnt lgkmcnt(" #n ")\n\t"
__device__ __forceinline__ void qk_hd256(f32x16& s0, f32x16& s1, const bf16x8 (&q)[2][16],
                                         const uint32_t (&ka)[8]) {
#if defined(__HIP_DEVICE_COMPILE__)
  bf16x8 t0, t1, t2;
  asm volatile(
      "s_nop 1\n\t"
      RA_KREAD(t0, a0, 0) RA_KREAD(t1, a1, 0)
      RA_KREAD(t2, a2, 0) RA_WAIT(2) RA_QK2(t0, 0, "0", "0")
      RA_KREAD(t0, a3, 0) RA_WAIT(2) RA_QK(t1, 1)
      RA_KREAD(t1, a4, 0) RA_WAIT(2) RA_QK(t2, 2)
      RA_KREAD(t2, a5, 0) RA_WAIT(2) RA_QK(t0, 3)
      RA_KREAD(t0, a6, 0) RA_WAIT(2) RA_QK(t1, 4)
      RA_KREAD(t1, a7, 0) RA_WAIT(2) RA_QK(t2, 5)
      RA_KREAD(t2, a0, 256) RA_WAIT(2) RA_QK(t0, 6)
      RA_KREAD(t0, a1, 256) RA_WAIT(2) RA_QK(t1, 7)
      RA_KREAD(t1, a2, 256) RA_WAIT(2) RA_QK(t2, 8)
      RA_KREAD(t2, a3, 256) RA_WAIT(2) RA_QK(t0, 9)
      RA_KREAD(t0, a4, 256) RA_WAIT(2) RA_QK(t1, 10)
      RA_KREAD(t1, a5, 256) RA_WAIT(2) RA_QK(t2, 11)
      RA_KREAD(t2, a6, 256) RA_WAIT(2) RA_QK(t0, 12)
      RA_KREAD(t0, a7, 256) RA_WAIT(2) RA_QK(t1, 13)
      RA_WAIT(1) RA_QK(t2, 14)
      RA_WAIT(0) RA_QK(t0, 15)
      "s_nop 7\n\t"
      "s_nop 7"
      : [s0] "=&v"(s0), [s1] "=&v"(s1), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2)
      : [q0_0] "v"(q[0][0]), [q0_1] "v"(q[0][1]), [q0_2] "v"(q[0][2]), [q0_3] "v"(q[0][3]),
        [q0_4] "v"(q[0][4]), [q0_5] "v"(q[0][5]), [q0_6] "v"(q[0][6]), [q0_7] "v"(q[0][7]),
        [q0_8] "v"(q[0][8]), [q0_9] "v"(q[0][9]), [q0_10] "v"(q[0][10]), [q0_11] "v"(q[0][11]),
        [q0_12] "v"(q[0][12]), [q0_13] "v"(q[0][13]), [q0_14] "v"(q[0][14]),
        [q0_15] "v"(q[0][15]),
        [q1_0] "v"(q[1][0]), [q1_1] "v"(q[1][1]), [q1_2] "v"(q[1][2]), [q1_3] "v"(q[1][3]),
        [q1_4] "v"(q[1][4]), [q1_5] "v"(q[1][5]), [q1_6] "v"(q[1][6]), [q1_7] "v"(q[1][7]),
        [q1_8] "v"(q[1][8]), [q1_9] "v"(q[1][9]), [q1_10] "v"(q[1][10]), [q1_11] "v"(q[1][11]),
        [q1_12] "v"(q[1][12]), [q1_13] "v"(q[1][13]), [q1_14] "v"(q[1][14]),
        [q1_15] "v"(q[1][15]),
        [a0] "v"(ka[0]), [a1] "v"(ka[1]), [a2] "v"(ka[2]), [a3] "v"(ka[3]), [a4] "v"(ka[4]),
        [a5] "v"(ka[5]), [a6] "v"(ka[6]), [a7] "v"(ka[7])
      : "memory");
#endif
}
#undef RA_KREAD
#undef RA_QK2
#undef RA_QK
#undef RA_WAIT

struct True { static constexpr bool value = true; };
struct False { static constexpr bool value = false; };

template <int D, bool F32OUT>
__global__ __launch_bounds__(kWaves * 64, 1) void ring_attn_fused_kernel(FusedParams p) {
  constexpr int NRB = kRowsPerWave / 32;  // 32-row MFMA blocks per wave
  constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  constexpr int NDB = D / 32;             // 32-wide d blocks of the output
  constexpr int NKS = D / 16;             // k-steps of the QK^T contraction
  constexpr int NKX = NKS < 8 ? NKS : 8;  // distinct K read patterns
  constexpr int NKB = kBKV / 32;          // 32-key blocks per tile
  constexpr int NPS = kBKV / 16;          // 16-key steps of P.V per tile
  constexpr int TILE = kBKV * D;          // elements of one K or V tile
  constexpr int DPW = kBKV * CPR / (64 * kWaves);  // DMA instructions per wave per tile
  static_assert(DPW >= 1 && DPW * 64 * kWaves == kBKV * CPR, "tile must split over the waves");
  // LDS: two K slots then two V slots.
  constexpr int NSLOT = 2;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * NSLOT * TILE];
  uint16_t* const kslot0 = lds;
  uint16_t* const vslot0 = lds + NSLOT * TILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int h = lane >> 5;   // lane half: keys / d interleave of the MFMA layouts
  const int lr = lane & 31;  // this lane's row within each 32-row block

  // XCD-aware workgroup order (grid is a multiple of 8).
  const int nwg = gridDim.x;
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nwg >> 3) + (bid >> 3);
  if (logical >= p.grid_real) return;
  const int g = logical / p.row_tiles;
  const int rt = p.row_tiles - 1 - (logical - g * p.row_tiles);  // long causal rows first
  const int row0 = rt * kRowsPerWG;

  // This lane's rows, one per row block.
  int token[NRB], head[NRB];
  bool row_ok[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = row0 + wave * kRowsPerWave + rb * 32 + lr;
    token[rb] = row / p.group;
    head[rb] = g * p.group + (row - token[rb] * p.group);
    row_ok[rb] = token[rb] < p.real_rows;
  }

  // Q^T operands: lane holds d = 16 s + 8 h + [0, 8) of each of its rows.
  // Loaded through a descriptor bounded at the real rows (rows past read 0).
  bf16x8 qreg[NRB][NKS];
  {
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc(p.q, (uint32_t)p.real_rows * (uint32_t)p.nq * D * 2);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const uint32_t qoff = ((uint32_t)token[rb] * p.nq + head[rb]) * D * 2 + 16 * h;
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        qreg[rb][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + 32 * s, 0, 0));
    }
  }

  // Tile schedule: ring region = P shard visits of nb tiles, then the
  // current tiles up to this workgroup's last real token.
  const int wg_last = min(p.real_rows - 1, (row0 + kRowsPerWG - 1) / p.group);
  const int wg_first = row0 / p.group;
  const int n_ring = p.P * p.nb;
  const int n_cur = wg_last / kBKV + 1;
  const int T = n_ring + n_cur;
  const uint32_t rowstride = (uint32_t)p.nkv * D * 2;  // bytes between tokens
  const uint32_t cur_bytes = (uint32_t)p.real_rows * rowstride;
  const int full_i = (int)p.full * p.interleave;  // < 2^31: bounded by a shard's length

  // Per-tile source, chosen by value: descriptors of the region (sized to
  // its valid rows), the tile's first byte, and the key bound.
  struct Src {
    i32x4 kr, vr;
    uint32_t off;     // byte offset of the tile's first row
    int lim_ring;     // ring: valid keys of the shard left from this tile
    int key0;         // current: chunk position of the tile's first key
    bool in_ring;
  };
  auto source = [&](int v) {
    Src s;
    s.in_ring = v < n_ring;
    if (v >= T) {  // past the walk: a zero-size fetch (fills the slot with zeros)
      s.kr = s.vr = make_desc(p.k_cur, 0);
      s.off = 0;
      s.lim_ring = 0;
      s.key0 = 0;
      s.in_ring = false;
      return s;
    }
    if (s.in_ring) {
      const int k = v / p.nb;
      const int b = v - k * p.nb;
      int sh = p.ring_start - k;
      sh += (sh < 0) ? p.P : 0;
      const int len = full_i + min(max((int)p.rem - sh * p.interleave, 0), p.interleave);
      const int64_t base = ((int64_t)sh * p.shard_cap * p.nkv + g) * D;
      const uint32_t bytes = (uint32_t)len * rowstride;
      s.kr = make_desc(p.k_cache + base, bytes);
      s.vr = make_desc(p.v_cache + base, bytes);
      s.off = (uint32_t)b * kBKV * rowstride;
      s.lim_ring = len - b * kBKV;
      s.key0 = 0;
    } else {
      const int c = v - n_ring;
      s.kr = make_desc(p.k_cur + g * D, cur_bytes);
      s.vr = make_desc(p.v_cur + g * D, cur_bytes);
      s.off = (uint32_t)c * kBKV * rowstride;
      s.lim_ring = 0;
      s.key0 = c * kBKV;
    }
    return s;
  };

  // DMA: wave-instruction i of this wave fills physical chunks
  // [(wave*DPW + i)*64, +64) of a tile, lane L the chunk at +L; the lane
  // fetches the logical chunk that the swizzle stores there.  The swizzles
  // permute row bits, so for the instruction's first row R (uniform) and
  // the lane's row r within it (disjoint bits) swz(R + r) = swz(R) ^ swz(r):
  // the lane offset is a per-lane base XOR a uniform term, and R's rows go
  // into the scalar offset.
  constexpr int RPI = 64 / CPR;  // tile rows per DMA instruction
  static_assert(RPI >= 1 && (RPI & (RPI - 1)) == 0, "rows per DMA instruction");
  const int dma_r = lane / CPR, dma_pc = lane % CPR;
  const uint32_t dma_kbase =
      (uint32_t)dma_r * rowstride + (uint32_t)((dma_pc ^ swz_k(dma_r, CPR)) << 4);
  const uint32_t dma_vbase =
      (uint32_t)dma_r * rowstride + (uint32_t)((dma_pc ^ swz_v(dma_r, CPR)) << 4);
  auto issue_k = [&](const Src& s, uint16_t* dst) {
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int R = (wave * DPW + i) * RPI;
      dma16(s.kr, dst + (wave * DPW + i) * 512, dma_kbase ^ (uint32_t)(swz_k(R, CPR) << 4),
            s.off + (uint32_t)R * rowstride);
    }
  };
  auto issue_v = [&](const Src& s, uint16_t* dst) {
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int R = (wave * DPW + i) * RPI;
      dma16(s.vr, dst + (wave * DPW + i) * 512, dma_vbase ^ (uint32_t)(swz_v(R, CPR) << 4),
            s.off + (uint32_t)R * rowstride);
    }
  };

  // K operand reads: lane reads row 32 kb + lr, chunk 2s + h.  (2s + h) ^ swz
  // = 2s ^ x with x = h ^ swz < 16, so steps s and s + 8 differ by 256 bytes
  // and key blocks by 32 rows.
  uint32_t kx[NKX];
  {
    const int x = h ^ swz_k(lr, CPR);
#pragma unroll
    for (int j = 0; j < NKX; ++j) kx[j] = (uint32_t)(lr * D * 2 + (((2 * j) ^ x) << 4));
  }
  // Transposed V reads.  Lane (block b4 = lane/16, i16 = lane%16) supplies
  // row 4h + i16/4 (+8 for the second half of the 8 keys, +16 per k-step)
  // and columns 32 db + 16 (b4 & 1) + 4 (i16 & 3); it receives d =
  // 32 db + 16 (b4 & 1) + i16 for 4 consecutive keys.  The d-block enters
  // the chunk index as 4 db, i.e. the byte offset as XOR (db << 6).
  uint32_t vbase;
  {
    const int b4 = lane >> 4, i16 = lane & 15;
    const int r = 4 * h + (i16 >> 2);
    const int c0 = 2 * (b4 & 1) + ((i16 & 3) >> 1);  // chunk within the 32-col block
    vbase = (uint32_t)(r * D * 2 + ((c0 ^ swz_v(r, CPR)) << 4) + 8 * (i16 & 1));
  }

  f32x16 acc[NRB][NDB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[rb][db] = f32x16{};
  float mlog[NRB], lsum[NRB], lsum_q[NRB];  // running max (log2 units), row sums
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    mlog[rb] = kNegInf;
    lsum[rb] = 0.f;     // exact fp32 sum of this lane's share of the keys
    lsum_q[rb] = 0.f;   // the same over bf16-rounded probabilities (fp32 output)
  }
  const float c2 = p.scale_log2e;

  // S^T = K Q^T for one tile: every K operand read from LDS feeds the MFMAs
  // of all NRB row blocks.  Operands are read two k-steps ahead and the
  // schedule alternates one LDS read with the MFMAs of one step (at
  // HD = 256 as one asm block, the scores in VGPRs).
  auto qk = [&](const uint16_t* kt, f32x16 (&S)[NRB][NKB]) {
    static_assert(NKB == 1, "one 32-key block per tile");
    if constexpr (D == 256 && NRB == 2) {
      const uint32_t k0 = (uint32_t)(uintptr_t)kt;  // LDS offset of the slot
      uint32_t ka[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ka[j] = kx[j] + k0;
      qk_hd256(S[0][0], S[1][0], qreg, ka);
    } else {
      auto kop = [&](int s) { return lds_read_b128(kt, kx[s & 7] + (s >> 3) * 256); };
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) S[rb][0] = f32x16{};
      bf16x8 ka[3];
      ka[0] = kop(0);
      ka[1] = kop(1);
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        if (s + 2 < NKS) ka[(s + 2) % 3] = kop(s + 2);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          S[rb][0] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s % 3], qreg[rb][s], S[rb][0], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the first two LDS reads
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        if (s + 2 < NKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, NRB, 0);                 // NRB MFMAs
      }
    }
  };

  // O^T += V^T P^T for one tile: every V operand feeds all row blocks.
  auto pv = [&](const uint16_t* vt, const bf16x8 (&pb)[NRB][NPS]) {
#pragma unroll
    for (int ks = 0; ks < NPS; ++ks) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint32_t o = (vbase ^ (uint32_t)(db << 6)) + ks * 16 * D * 2;
        const i16x4 x1 = lds_read_tr(vt, o);
        const i16x4 x2 = lds_read_tr(vt, o + 8 * D * 2);
        const i16x8 x = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
        const bf16x8 a = __builtin_bit_cast(bf16x8, x);
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          acc[rb][db] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[rb][ks], acc[rb][db], 0, 0, 0);
      }
    }
  };

  // Region by value: keys with index >= lim[rb] in the tile are masked.
  auto mask = [&](f32x16 (&S)[NRB][NKB], const int (&lim)[NRB]) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + (i >> 2) * 8 + 4 * h + (i & 3);
          S[rb][kb][i] = key < lim[rb] ? S[rb][kb][i] : kNegInf;
        }
  };

  // Online softmax of one tile, in place: S becomes the probabilities
  // (fp32).  alpha[rb] is the factor the accumulator must be scaled by (1
  // unless some row of the wave raised its running max by more than kTau;
  // the return value reports whether any did).  lsum is the exact fp32 row
  // sum (for the LSE and, with bf16 output, the normalisation); for fp32
  // output the normalisation uses lsum_q instead (see pack).
  auto softmax = [&](f32x16 (&S)[NRB][NKB], float (&alpha)[NRB]) {
    bool any = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2)
          mx = __builtin_elementwise_maximum(
              mx, __builtin_elementwise_maximum(S[rb][kb][i], S[rb][kb][i + 1]));
      mx = wave_max_pair(mx) * c2;  // scale > 0, so max commutes with the scaling
      const bool need = mx > mlog[rb] + kTau<F32OUT>;
      const bool anyrb = __builtin_amdgcn_ballot_w64(need) != 0;
      const float m_new = anyrb ? __builtin_elementwise_maximum(mlog[rb], mx) : mlog[rb];
      alpha[rb] = (m_new == mlog[rb]) ? 1.f : __builtin_amdgcn_exp2f(mlog[rb] - m_new);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          S[rb][kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[rb][kb][i], c2, -m_use));
          ls += S[rb][kb][i];
        }
      lsum[rb] = lsum[rb] * alpha[rb] + ls;
      mlog[rb] = m_new;
      any |= anyrb;
    }
    return any;
  };
  // Probabilities -> bf16 B operands of P.V.  For fp32 output also the sum
  // of the bf16-rounded probabilities (v_dot2 against (1, 1)): numerator
  // and denominator then weight every key identically.
  auto pack = [&](const f32x16 (&S)[NRB][NKB], bf16x8 (&pb)[NRB][NPS], const float (&alpha)[NRB]) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float lq = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const bf16x2 pr = {(__bf16)S[rb][kb][i], (__bf16)S[rb][kb][i + 1]};
          if (F32OUT) lq = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lq, false);
          pb[rb][2 * kb + (i >> 3)][i & 7] = pr[0];
          pb[rb][2 * kb + (i >> 3)][(i & 7) + 1] = pr[1];
        }
      if (F32OUT) lsum_q[rb] = lsum_q[rb] * alpha[rb] + lq;
    }
  };

  // Region by value: each row's key bound within the tile, and whether any
  // bound of the workgroup cuts into the tile (then the compare is needed).
  auto bounds = [&](const Src& src, int (&lim)[NRB]) {
    if (src.in_ring) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) lim[rb] = src.lim_ring;
      return src.lim_ring < kBKV;
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) lim[rb] = token[rb] + 1 - src.key0;
    return src.key0 + kBKV > wg_first + 1;
  };

  // Iteration v reads K(v) and V(v-1) and fetches K(v+1) and V(v) into the
  // slots that K(v-1) and V(v-2) left.  The scores of tile v are computed,
  // then its softmax is issued between the P.V MFMAs of tile v-1, which do
  // not depend on it, then tile v's bf16 packing; the rare rescale for tile
  // v's max is applied at the top of the next iteration, between P.V(v-1)
  // and P.V(v).  The accumulator is touched by no branch but the rescale.
  Src s0 = source(0), s1 = source(1);  // tiles v, v+1
  issue_k(s0, kslot0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
  __syncthreads();

  bf16x8 pb[NRB][NPS];
  bool any = false;       // the previous tile asked for a rescale ...
  float alpha[NRB];       // ... by these factors
  auto rescale = [&]() {
    if (any) {
#if defined(__HIP_DEVICE_COMPILE__)
      // the last P.V MFMAs may still be writing acc: wait them out
      asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#endif
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) scale_agprs(acc[rb][db], alpha[rb]);
    }
  };
  int sl = 0;  // LDS slot of tile v
  // Issue the copies of K(v+1) and V(v), compute tile v's scores, mask them.
  auto front = [&](f32x16 (&S)[NRB][NKB]) {
    issue_k(s1, kslot0 + (sl ^ 1) * TILE);
    issue_v(s0, vslot0 + sl * TILE);
    qk(kslot0 + sl * TILE, S);
    int lim[NRB];
    if (bounds(s0, lim)) mask(S, lim);
  };
  auto advance = [&](int v) {
    s0 = s1;
    s1 = source(v + 2);
    sl ^= 1;
  };
  {  // tile 0: no P.V yet
    f32x16 S[NRB][NKB];
    front(S);
    any = softmax(S, alpha);
    pack(S, pb, alpha);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K(1), V(0) have landed
    __syncthreads();
    advance(0);
  }
  // P.V of the previous tile with the softmax of the current one, hand
  // ordered: slot t issues the MFMAs of P.V step t (one V operand, read two
  // slots ahead, for every row block) and then a fixed slice of softmax
  // work; sched_barrier keeps slices in their slots so the VALU and
  // transcendental work runs under the MFMAs.  Softmax work units, in
  // dependency order: the in-lane max of each row block, the cross-lane
  // reduction and new running max, one exp2 per score, the row sums.
  auto pv_softmax = [&](const uint16_t* vt, f32x16 (&S)[NRB][NKB], float (&al)[NRB]) {
    constexpr int NT = NPS * NDB;                  // P.V steps
    constexpr int NE = NRB * NKB * 16;              // exp2 units
    constexpr int NU = NRB + 1 + NE + 1;            // all units
    auto vop = [&](int t) {
      const int ks = t / NDB, db = t % NDB;
      const uint32_t o = (vbase ^ (uint32_t)(db << 6)) + ks * 16 * D * 2;
      const i16x4 x1 = lds_read_tr(vt, o);
      const i16x4 x2 = lds_read_tr(vt, o + 8 * D * 2);
      const i16x8 x = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
      return __builtin_bit_cast(bf16x8, x);
    };
    float mx[NRB], m_use[NRB], ls[NRB];
    bool any = false;
    auto unit = [&](int u) {
      if (u < NRB) {  // in-lane max of row block u
        float m = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; i += 2)
            m = __builtin_elementwise_maximum(
                m, __builtin_elementwise_maximum(S[u][kb][i], S[u][kb][i + 1]));
        mx[u] = m;
      } else if (u == NRB) {  // cross-lane max, vote, new running max
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const float m = wave_max_pair(mx[rb]) * c2;  // scale > 0: max commutes
          const bool need = m > mlog[rb] + kTau<F32OUT>;
          const bool anyrb = __builtin_amdgcn_ballot_w64(need) != 0;
          const float m_new = anyrb ? __builtin_elementwise_maximum(mlog[rb], m) : mlog[rb];
          al[rb] = (m_new == mlog[rb]) ? 1.f : __builtin_amdgcn_exp2f(mlog[rb] - m_new);
          m_use[rb] = m_new == kNegInf ? 0.f : m_new;
          mlog[rb] = m_new;
          ls[rb] = 0.f;
          any |= anyrb;
        }
      } else if (u < NRB + 1 + NE) {  // one probability
        const int q = u - NRB - 1;
        const int rb = q / (NKB * 16), kb = (q / 16) % NKB, i = q % 16;
        S[rb][kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[rb][kb][i], c2, -m_use[rb]));
        ls[rb] += S[rb][kb][i];
      } else {  // row sums
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) lsum[rb] = lsum[rb] * al[rb] + ls[rb];
      }
    };
    bf16x8 va[3];
    va[0] = vop(0);
    if (NT > 1) va[1] = vop(1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int ks = t / NDB, db = t % NDB;
      if (t + 2 < NT) va[(t + 2) % 3] = vop(t + 2);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        acc[rb][db] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t % 3], pb[rb][ks], acc[rb][db], 0, 0, 0);
      // units [t*NU/NT, (t+1)*NU/NT), the rest after the last slot
#pragma unroll
      for (int u = t * NU / NT; u < (t + 1) * NU / NT; ++u) unit(u);
      __builtin_amdgcn_sched_barrier(0);
    }
    return any;
  };
  for (int v = 1; v < T; ++v) {
    rescale();
    f32x16 S[NRB][NKB];
    front(S);
    any = pv_softmax(vslot0 + (sl ^ 1) * TILE, S, alpha);
    pack(S, pb, alpha);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K(v+1), V(v) have landed
    __syncthreads();
    advance(v);
  }
  rescale();
  pv(vslot0 + (sl ^ 1) * TILE, pb);

  // Epilogue: out = acc / l, lse = ln 2 * (m + log2 l).
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float l_tot = lsum[rb] + __shfl_xor(lsum[rb], 32);
    const float l_norm = F32OUT ? lsum_q[rb] + __shfl_xor(lsum_q[rb], 32) : l_tot;
    if (!row_ok[rb]) continue;
    const float inv = 1.f / l_norm;
    const int64_t obase = ((int64_t)token[rb] * p.nq + head[rb]) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = db * 32 + i4 * 8 + 4 * h;
        const f32x4 o = {acc[rb][db][4 * i4] * inv, acc[rb][db][4 * i4 + 1] * inv,
                         acc[rb][db][4 * i4 + 2] * inv, acc[rb][db][4 * i4 + 3] * inv};
        if (F32OUT) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + obase + d0) = o;
        } else {
          const bf16x4 ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
          *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.out) + obase + d0) = ob;
        }
      }
    }
    if (h == 0 && p.lse != nullptr)
      p.lse[(int64_t)head[rb] * p.q_rows + token[rb]] = (mlog[rb] + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace

template <int D>
static void launch_hd(const FusedParams& p, dim3 grid, dim3 block, hipStream_t stream) {
  if (p.out_f32)
    hipLaunchKernelGGL((ring_attn_fused_kernel<D, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((ring_attn_fused_kernel<D, false>), grid, block, 0, stream, p);
}

hipError_t launch_fused(const FusedParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid((p.grid_real + 7) / 8 * 8);
  const dim3 block(kWaves * 64);
  switch (head_dim) {
    case 64: launch_hd<64>(p, grid, block, stream); break;
    case 128: launch_hd<128>(p, grid, block, stream); break;
    case 256: launch_hd<256>(p, grid, block, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ra
