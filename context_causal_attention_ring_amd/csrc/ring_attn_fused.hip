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
//    accumulator (64 rows x HD) lives in the AGPRs; at HD = 256 each tile is
//    one hand-scheduled asm block (tile_hd256.inc, see tile_hd256 below),
//    and at HD = 128 and 64 with bf16 output one asm block per step works
//    on three tiles: the scores of tile u, the softmax of tile u-1 and the
//    P.V of tile u-2 (tile_hd128.inc, tile_hd64.inc, see tile_pipe below).
//  * K/V tiles of 32 keys go HBM -> LDS by buffer_load ... lds (no register
//    staging) into four K and four V slots (tile t in slot t mod 4).  Tiles
//    run in pairs with one wait and one barrier per pair; while a pair is
//    computed, the copies of the next pair (K two tiles ahead, V one tile
//    behind it) are in flight, issued between the score MFMAs.  Their
//    sources, and each tile's key bound, come from three scalar walkers
//    (region descriptor, tile offset, bound, tiles left) that step with two
//    adds and build a descriptor only on entering the next region.
//    Rows are stored with a 16-byte-chunk XOR swizzle chosen per operand so
//    that K reads (32 rows, one chunk) and transposed V reads
//    (ds_read_b64_tr_b16, 4 rows x 4 chunks) are both bank-conflict free at
//    HD = 256 and 128.  At HD = 64 a row has 8 chunks and the K reads meet
//    some conflicts; they wait behind the MFMAs (a conflict-free pattern
//    for that case timed no faster).
//  * Fetches go through buffer descriptors whose size is the valid length
//    of the visited region: rows past a shard's length (or past the real
//    chunk rows) come back as zeros without touching memory -- the
//    zero-size fetch of the inactive region, chosen by value.  The mask is
//    one bound per row, key < lim, with lim = shard length in the ring
//    region and token + 1 (causal) in the current region; tiles that no
//    bound cuts skip the compare entirely.
//  * Online softmax in log2 units with a lazy running max: a 32-row block
//    of the accumulator is rescaled only when some row of it raised its max
//    by more than kTau (a vote), so the common tile costs fma, exp2, add and
//    a bf16 pack per score.  The softmax of tile v is issued between the
//    P.V MFMAs of tile v-1, which do not depend on it, in a hand-ordered
//    block (one MFMA pair, one V operand read, a slice of softmax work); in
//    the three-tile blocks between all the MFMAs of the next step, whose
//    score MFMAs write the other of two score buffers.
//  * P.V takes bf16 weights.  bf16 output is normalised by the fp32 row sum
//    corrected, for every tile that holds a sizeable share of a row's
//    weight, by the rounding of that tile's weights, so numerator and
//    denominator weight its keys identically; fp32 output feeds P.V each
//    weight as a bf16 pair hi + lo (two MFMAs per step).
//  * With the strided cache write fused in (ring_attn_prefill_write), each
//    workgroup copies its share of the chunk's tokens into their cache
//    slots after its epilogue; the walk never reads those slots.
//  * Workgroup ids are remapped so that the workgroups resident on one XCD
//    share a KV head and walk the same tiles, keeping the re-streamed K/V in
//    that XCD's L2, with the KV head's row tiles dealt to its XCDs in turn,
//    longest causal rows first.
#include "ra_internal.h"

namespace ra {
namespace {

// Lambdas of the kernel are inlined: their captures must stay in registers.
#define RA_INLINE __attribute__((always_inline))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
// Lazy-rescale threshold (log2 units): probabilities stay <= 2^kTau.  The
// P.V product never sees a weight rounded relative to another: with bf16
// output the output is normalised by the sum of the same bf16-rounded
// probabilities the MFMAs take; with fp32 output each probability enters
// P.V as a bf16 pair hi + lo that holds it to about 2^-16.
template <bool F32OUT>
constexpr float kTau = 8.0f;
// With bf16 output the tile blocks first take each tile's scores against
// the running max as it stands; a lane whose 16 probabilities sum to more
// than 2^kTau may hold one above 2^kTau, and then the block recomputes the
// tile with the max updated (at HD = 256 from its K slot, in the three-tile
// blocks from the scores they kept).
constexpr float kPBound = 256.0f;  // 2^kTau<false>

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
  // the descriptor and the scalar offset are wave-uniform by construction;
  // readfirstlane keeps them in SGPRs where the analysis cannot prove it
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  const i32x4 r = {__builtin_amdgcn_readfirstlane(rs[0]), __builtin_amdgcn_readfirstlane(rs[1]),
                   __builtin_amdgcn_readfirstlane(rs[2]), __builtin_amdgcn_readfirstlane(rs[3])};
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(m0), "v"(voff), "s"(r), "s"(so)
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

// One 32-key tile at HD = 256 as a single instruction block (generated:
// tile_hd256.inc; this binds its operands).  In order: S^T = K Q^T of tile
// v from the K slot at KOFF, its first two operands already in kpre; if a
// key bound cuts the tile (the counter nm below ran out), scores of keys at
// or past each row's bound become -inf; then O^T += V^T P^T of tile v-1 (V slot at VOFF, bf16
// probabilities pin) with tile v's online softmax in the MFMAs' shadow.  The
// even tile of a pair (PIN = 1) reads the odd tile's kpre from the K slot at
// KPO during its P.V; the odd tile (PIN = 0) ends with the pair's wait for
// this wave's copies and barrier, then reads the next pair's kpre (slot KPO)
// and leaves it in flight (the next block waits for it).  On return pout
// holds tile v's bf16 probabilities, ml the updated running max (log2
// units), lo / lko the row sums li / lki with this tile folded in (the
// caller alternates two register sets by tile parity, so a slow path
// still finds li as it was), al the factor the accumulator must be scaled by, and
// bit rb of resc is set when some row of row block rb asked for that
// rescale (al == 1 for every row of the other blocks).
//   ka[j]  LDS address of this lane's K row at chunk (2j + h) ^ swizzle;
//          k-step s reads ka[s % 8] + KOFF + 256 (s / 8)
//   va[d]  LDS address of this lane's transposed V read for d blocks d and
//          d + 4; step (ks, db) reads va[db % 4] + VOFF + 8192 ks + 256
//          (db / 4), and + 4096 for keys 8..15
// Q and the two probability buffers are pinned to v[44:203] (buffer PIN is
// read, 1 - PIN written) and kpre to v[236:243]; scores live in v[204:235]
// and the operand ring in v[244:255] (clobbered).
// The block also issues this wave's LDS-DMA copies of one K tile (source
// desck at tile offset offk, to the slot at MK) and one V tile (descv, offv,
// to MV), four instructions each.  Instruction j = 2 a + b of wave w moves
// rows 2 w + 8 a + 16 b and the next (to LDS m0b + 512 (8 a + 16 b) past the
// slot); its lane offset is dl.ka / dl.kb (dl.va / dl.vb) for a = 0 / 1, and
// b adds dl.rs16, 16 rows' stride, to the scalar offset.  The caller waits
// for them (vmcnt) and synchronises before the slots are read.
// It then steps the walkers to the next tile in the same shadow: offk and
// offv by tstr (one tile), the bound walker's wlim by dlim, and the two
// counters the caller keeps by one: nm, the tiles before the next one a key
// bound cuts (this tile is cut when nm was 0 or below: the mask above), and
// tn, the tiles before some walker enters its next region (at 0 the caller
// takes the walkers there).
#include "tile_hd256.inc"
#define RA_TILE_STATE_OPERANDS                                                                  \
  [ml0] "+v"(ml[0]), [ml1] "+v"(ml[1]), [lo0] "=&v"(lo[0]), [lo1] "=&v"(lo[1]),                 \
      [lko0] "=&v"(lko[0]), [lko1] "=&v"(lko[1]), [al0] "=&v"(al[0]), [al1] "=&v"(al[1]),      \
      [resc] "=&s"(resc), [any] "=&s"(any), [a0] "=&v"(a0), [b0] "=&v"(b0), [a1] "=&v"(a1),    \
      [b1] "=&v"(b1), [th0] "=&v"(th0), [th1] "=&v"(th1), [r0] "=&v"(r0), [r1] "=&v"(r1),      \
      [c0] "=&s"(c0), [c1] "=&s"(c1), [v0] "=&s"(v0), [v1] "=&s"(v1), [st] "=&s"(st),          \
      [lc] "=&s"(lc), [lm] "=&s"(lm), [wt] "=&s"(wt), [offk] "+s"(offk), [offv] "+s"(offv),   \
      [wlim] "+s"(wlim), [nm] "+s"(nm), [tn] "+s"(tn)
// bf16 output: the rounded-minus-fp32 sums of the significant tiles, and
// the tile-sum bound past which a tile is significant
#define RA_TILE_LQ_OPERANDS                                                                     \
  [dq0] "+v"(dq[0]), [dq1] "+v"(dq[1]), [bnd0] "+v"(bnd[0]), [bnd1] "+v"(bnd[1])
#define RA_TILE_INPUT_OPERANDS                                                                  \
  [ka0] "v"(ka[0]), [ka1] "v"(ka[1]), [ka2] "v"(ka[2]), [ka3] "v"(ka[3]), [ka4] "v"(ka[4]),    \
      [ka5] "v"(ka[5]), [ka6] "v"(ka[6]), [ka7] "v"(ka[7]), [va0] "v"(va[0]), [va1] "v"(va[1]), \
      [va2] "v"(va[2]), [va3] "v"(va[3]), [c2] "s"(c2), [tau] "s"(tau), [pbnd] "s"(pbnd),       \
      [wk] "s"(wb.k), [li0] "v"(li[0]), [li1] "v"(li[1]), [lki0] "v"(lki[0]),                   \
      [lki1] "v"(lki[1]), [np] "s"(wb.np), [dlim] "s"(dlim), [vv] "s"(wb.v), [tt] "s"(wb.t),   \
      [pos0] "v"(pos[0]), [pos1] "v"(pos[1]),                                                  \
      [ninf] "v"(ninf), [kpo] "i"(KPO), [desck] "s"(desck), [descv] "s"(descv),                 \
      [tstr] "s"(tstr), [m0b] "s"(m0b), [rs16] "s"(dl.rs16)
// l <- l * a + r, compensated (Kahan summation): c holds the part of the
// sum that earlier folds rounded away (negated), and the fold adds it back,
// so a row sum over millions of keys whose tile sums are tiny against it
// (a peaky row: one dominant key, the rest near 0) does not drift.  The
// sum's best value is l - c.  Contraction stays off: t - lp must see the
// rounded product.
__device__ __forceinline__ void fold_sum(float& l, float& c, float a, float r) {
#pragma clang fp contract(off)
  const float lp = l * a;
  const float y = r - c * a;
  const float t = lp + y;
  c = (t - lp) - y;
  l = t;
}

struct TileBound {    // what a cut tile's key bound comes from (uniform)
  int k, np;          // the tile's region and P (k >= P: current tiles)
  int v, t;           // the tile and the walk's length (v >= t: past the walk)
};

struct CopyLanes {    // a lane's offsets for the block's LDS-DMA copies (see below)
  uint32_t ka, kb, va, vb;
  uint32_t rs16;      // 16 rows' stride in bytes (uniform)
};
template <bool F32, uint32_t KOFF, uint32_t VOFF, int PIN, uint32_t MK, uint32_t MV,
          uint32_t KPO>
__device__ __forceinline__ void tile_hd256(f32x16 (&acc)[2][8], bf16x8 (&p0)[2][2],
                                           bf16x8 (&p1)[2][2], const bf16x8 (&q)[2][16],
                                           bf16x8 (&kpre)[2], const uint32_t (&ka)[8],
                                           const uint32_t (&va)[4],
                                           float (&ml)[2], const float (&li)[2],
                                           const float (&lki)[2], float (&lo)[2], float (&lko)[2],
                                           float (&dq)[2], float (&bnd)[2], float (&al)[2],
                                           uint32_t& resc, float c2, float tau, float pbnd,
                                           const TileBound& wb, const int (&pos)[2],
                                           const i32x4& desck, const i32x4& descv,
                                           uint32_t& offk, uint32_t& offv, int& wlim, int dlim,
                                           int& nm, uint32_t& tn, uint32_t tstr, uint32_t m0b,
                                           const CopyLanes& dl) {
#if defined(__HIP_DEVICE_COMPILE__)
  float a0, b0, a1, b1, th0, th1, r0, r1;
  uint32_t st, lc, lm, wt, v0, v1;
  uint64_t c0, c1, any;
  const float ninf = kNegInf;
  const uint32_t one2 = 0x3F803F80u;   // bf16 pair (1, 1): v_dot2 sums a packed pair
  const uint32_t hmask = 0xFFFF0000u;  // the bf16 truncation of an fp32 word
  const uint32_t psel = 0x07060302u;   // v_perm: the upper halves of two words
  if constexpr (PIN == 0 && !F32) {
    asm volatile(RA_TILE_HD256_ASM_P0
                 : RA_TILE_STATE_OPERANDS, RA_TILE_HD256_ACC_OPERANDS, RA_TILE_HD256_KPRE_OPERANDS,
                   RA_TILE_LQ_OPERANDS, RA_TILE_HD256_PB_OUT1
                 : RA_TILE_HD256_Q_OPERANDS, RA_TILE_HD256_PB_IN0, RA_TILE_INPUT_OPERANDS,
                   RA_TILE_HD256_OFFSET_OPERANDS, [one2] "s"(one2)
                 : RA_TILE_HD256_CLOBBERS, "memory", "scc", "m0");
  } else if constexpr (!F32) {
    asm volatile(RA_TILE_HD256_ASM_P1
                 : RA_TILE_STATE_OPERANDS, RA_TILE_HD256_ACC_OPERANDS, RA_TILE_HD256_KPRE_OPERANDS,
                   RA_TILE_LQ_OPERANDS, RA_TILE_HD256_PB_OUT0
                 : RA_TILE_HD256_Q_OPERANDS, RA_TILE_HD256_PB_IN1, RA_TILE_INPUT_OPERANDS,
                   RA_TILE_HD256_OFFSET_OPERANDS, [one2] "s"(one2)
                 : RA_TILE_HD256_CLOBBERS, "memory", "scc", "m0");
  } else if constexpr (PIN == 0) {
    asm volatile(RA_TILE_HD256_F32_P0
                 : RA_TILE_STATE_OPERANDS, RA_TILE_HD256_ACC_OPERANDS, RA_TILE_HD256_KPRE_OPERANDS,
                   RA_TILE_HD256_PB_RW0, RA_TILE_HD256_PB_RW1
                 : RA_TILE_HD256_Q_OPERANDS, RA_TILE_INPUT_OPERANDS, RA_TILE_HD256_OFFSET_OPERANDS,
                   [hmask] "s"(hmask),
                   [psel] "s"(psel)
                 : RA_TILE_HD256_CLOBBERS, "memory", "scc", "m0");
  } else {
    asm volatile(RA_TILE_HD256_F32_P1
                 : RA_TILE_STATE_OPERANDS, RA_TILE_HD256_ACC_OPERANDS, RA_TILE_HD256_KPRE_OPERANDS,
                   RA_TILE_HD256_PB_RW0, RA_TILE_HD256_PB_RW1
                 : RA_TILE_HD256_Q_OPERANDS, RA_TILE_INPUT_OPERANDS, RA_TILE_HD256_OFFSET_OPERANDS,
                   [hmask] "s"(hmask),
                   [psel] "s"(psel)
                 : RA_TILE_HD256_CLOBBERS, "memory", "scc", "m0");
  }
#endif
}

// One step of the HD = 128 or HD = 64 tile loop (generated by
// gen_tile_pipe.py: tile_hd128.inc, tile_hd64.inc; this binds their
// operands).  Block u computes S^T = K Q^T of tile u (K slot at KOFF, first
// two operands in kpre) into score buffer sc[E], E = u mod 2; runs the
// online softmax of tile u-1 on sc[1 - E]; and accumulates O^T += V^T P^T
// of tile u-2 (V slot at VOFF).  bf16 output: the softmax of the HD = 256
// block (raw scores kept: the exponentials go to temporaries, so the slow
// path needs no second S^T; the significant-tile correction) into
// probability buffer 1 - E, while P.V reads buffer E.  fp32 output (F32):
// the exact-max softmax in place and hi + lo probabilities, single-buffered
// in p0 (hi) and p1 (lo) as in the HD = 256 fp32 block, four P.V MFMAs per
// step.  The softmax is spread over all the block's MFMAs.  When tile
// u is cut by a key bound its scores are masked at the end of the block,
// for the next one.  Copies: the wave's rows of K tile u + 2 (to MK) and V
// tile u (to MV), D / 64 instructions each; copy b of wave w moves the 1024
// / (2 D) rows from row (1024 / (2 D)) w + 16 b on, lane offset dl.ka /
// dl.va, and b = 1 adds dl.rs16 to the scalar offset.  The even block reads
// tile u + 1's kpre from KPO during its P.V; the odd block ends the pair
// (copies waited for, barrier) and leaves the next kpre in flight.  The
// walkers step as in the HD = 256 block.  On return ml, lo / lko, al and
// resc are those of tile u-1's softmax.
//   ka[j]  LDS address of this lane's K row at chunk (2j + h) ^ swizzle;
//          k-step s reads ka[s] + KOFF
//   va[d]  LDS address of this lane's transposed V read for d block d;
//          step (ks, db) reads va[db] + VOFF + 32 D ks, and + 16 D for keys
//          8..15
// HD = 128: Q is pinned to v[44:107], the score buffers to v[108:171], the
// probability buffers to v[172:203] and kpre to v[236:243]; the
// exponentials use v[204:211] and the operand ring v[244:255] (clobbered).
// HD = 64 runs two workgroups per CU (a wave has 256 registers, 64 of them
// the accumulator's): Q v[44:75], the score buffers v[76:139], the
// probability buffers v[140:171], the exponentials v[172:179] and the ring
// v[180:191]; there is no kpre: each block reads its first two K operands
// itself, and the other wave on the SIMD covers their latency.
#include "tile_hd128.inc"
#include "tile_hd64.inc"
#define RA_TILE_PIPE_ASM(HD, E, SOUT, SRW, POUT, PIN)                                          \
  asm volatile(RA_TILE_HD##HD##_E##E                                                            \
               : RA_TILE_STATE_OPERANDS, RA_TILE_HD##HD##_ACC_OPERANDS,                         \
                 RA_TILE_HD##HD##_KPRE_OPERANDS, RA_TILE_LQ_OPERANDS, RA_TILE_HD##HD##_##POUT,  \
                 RA_TILE_HD##HD##_##SOUT, RA_TILE_HD##HD##_##SRW                                \
               : RA_TILE_HD##HD##_Q_OPERANDS, RA_TILE_HD##HD##_##PIN, RA_TILE_INPUT_OPERANDS,   \
                 RA_TILE_HD##HD##_OFFSET_OPERANDS, [one2] "s"(one2)                             \
               : RA_TILE_HD##HD##_CLOBBERS, "memory", "scc", "m0")
// fp32 output: hi and lo probabilities both read and rewritten, no dq / bound
#define RA_TILE_PIPE_F32_ASM(HD, E, SOUT, SRW)                                                 \
  asm volatile(RA_TILE_HD##HD##_F32_E##E                                                        \
               : RA_TILE_STATE_OPERANDS, RA_TILE_HD##HD##_ACC_OPERANDS,                         \
                 RA_TILE_HD##HD##_KPRE_OPERANDS, RA_TILE_HD##HD##_PB_RW0,                       \
                 RA_TILE_HD##HD##_PB_RW1, RA_TILE_HD##HD##_##SOUT, RA_TILE_HD##HD##_##SRW        \
               : RA_TILE_HD##HD##_Q_OPERANDS, RA_TILE_INPUT_OPERANDS,                           \
                 RA_TILE_HD##HD##_OFFSET_OPERANDS, [hmask] "s"(hmask), [psel] "s"(psel)         \
               : RA_TILE_HD##HD##_CLOBBERS, "memory", "scc", "m0")
template <int D, bool F32, uint32_t KOFF, uint32_t VOFF, int E, uint32_t MK, uint32_t MV,
          uint32_t KPO>
__device__ __forceinline__ void tile_pipe(f32x16 (&acc)[2][D / 32], f32x16 (&sc)[2][2],
                                          bf16x8 (&p0)[2][2], bf16x8 (&p1)[2][2],
                                          const bf16x8 (&q)[2][D / 16], bf16x8 (&kpre)[2],
                                          const uint32_t (&ka)[8], const uint32_t (&va)[4],
                                          float (&ml)[2], const float (&li)[2],
                                          const float (&lki)[2], float (&lo)[2], float (&lko)[2],
                                          float (&dq)[2], float (&bnd)[2], float (&al)[2],
                                          uint32_t& resc, float c2, float tau, float pbnd,
                                          const TileBound& wb, const int (&pos)[2],
                                          const i32x4& desck, const i32x4& descv,
                                          uint32_t& offk, uint32_t& offv, int& wlim, int dlim,
                                          int& nm, uint32_t& tn, uint32_t tstr, uint32_t m0b,
                                          const CopyLanes& dl) {
  static_assert(D == 128 || D == 64, "three-tile blocks exist for HD 128 and 64");
#if defined(__HIP_DEVICE_COMPILE__)
  float a0, b0, a1, b1, th0, th1, r0, r1;
  uint32_t st, lc, lm, wt, v0, v1;
  uint64_t c0, c1, any;
  const float ninf = kNegInf;
  const uint32_t one2 = 0x3F803F80u;  // bf16 pair (1, 1): v_dot2 sums a packed pair
  const uint32_t hmask = 0xFFFF0000u;  // the bf16 truncation of an fp32 word
  const uint32_t psel = 0x07060302u;   // v_perm: the upper halves of two words
  [[maybe_unused]] uint32_t kpd = 0;    // HD = 64: stands in for kpre (nothing read ahead)
  if constexpr (F32 && D == 128 && E == 0) {
    RA_TILE_PIPE_F32_ASM(128, 0, S_OUT0, S_RW1);
  } else if constexpr (F32 && D == 128) {
    RA_TILE_PIPE_F32_ASM(128, 1, S_OUT1, S_RW0);
  } else if constexpr (F32 && E == 0) {
    RA_TILE_PIPE_F32_ASM(64, 0, S_OUT0, S_RW1);
  } else if constexpr (F32) {
    RA_TILE_PIPE_F32_ASM(64, 1, S_OUT1, S_RW0);
  } else if constexpr (D == 128 && E == 0) {
    RA_TILE_PIPE_ASM(128, 0, S_OUT0, S_RW1, PB_OUT1, PB_IN0);
  } else if constexpr (D == 128) {
    RA_TILE_PIPE_ASM(128, 1, S_OUT1, S_RW0, PB_OUT0, PB_IN1);
  } else if constexpr (E == 0) {
    RA_TILE_PIPE_ASM(64, 0, S_OUT0, S_RW1, PB_OUT1, PB_IN0);
  } else {
    RA_TILE_PIPE_ASM(64, 1, S_OUT1, S_RW0, PB_OUT0, PB_IN1);
  }
#endif
}
#undef RA_TILE_PIPE_ASM
#undef RA_TILE_PIPE_F32_ASM
#undef RA_TILE_STATE_OPERANDS
#undef RA_TILE_LQ_OPERANDS
#undef RA_TILE_INPUT_OPERANDS

template <int D, bool F32OUT>
__global__ __launch_bounds__(kWaves * 64, kWGsPerCU<D>) void ring_attn_fused_kernel(
    FusedParams p) {
  constexpr int NRB = kRowsPerWave / 32;  // 32-row MFMA blocks per wave
  constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
  constexpr int NDB = D / 32;             // 32-wide d blocks of the output
  constexpr int NKS = D / 16;             // k-steps of the QK^T contraction
  constexpr int NKX = NKS < 8 ? NKS : 8;  // distinct K read patterns
  constexpr int NKB = kBKV / 32;          // 32-key blocks per tile
  constexpr int NPS = kBKV / 16;          // 16-key steps of P.V per tile
  constexpr int TILE = kBKV * D;          // elements of one K or V tile
  constexpr uint32_t TILE_B = TILE * 2;   // bytes of one K or V tile
  constexpr int DPW = kBKV * CPR / (64 * kWaves);  // DMA instructions per wave per tile
  static_assert(DPW >= 1 && DPW * 64 * kWaves == kBKV * CPR, "tile must split over the waves");
  // hand-scheduled tile bodies: HD = 256 (one tile per block) and the
  // three-tile blocks at HD = 128 and 64, both output types
  constexpr bool ASM256 = D == 256 && NRB == 2 && NKB == 1;
  constexpr bool ASMPIPE = (D == 128 || D == 64) && NRB == 2 && NKB == 1;
  constexpr bool ASMBLK = ASM256 || ASMPIPE;
  // LDS: K slots 0..3 then V slots 0..3 (tile t in slot t mod 4).  Slot
  // offsets are compile-time constants because the tile loop is unrolled
  // over the four slots.
  constexpr int NSLOT = 4;
  constexpr uint32_t VBASE = NSLOT * TILE_B;  // byte offset of the V slots
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * NSLOT * TILE];
  auto kslot = [&](int s) RA_INLINE { return lds + s * TILE; };
  auto vslot = [&](int s) RA_INLINE { return lds + (NSLOT + s) * TILE; };
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;  // LDS byte address of the slots

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int h = lane >> 5;   // lane half: keys / d interleave of the MFMA layouts
  const int lr = lane & 31;  // this lane's row within each 32-row block

  // XCD-aware workgroup order (grid is a multiple of 8): workgroup bid runs
  // on XCD bid % 8, so XCD x takes the logical items [x, x + 1) * nwg / 8.
  const int nwg = gridDim.x;
  const int bid = blockIdx.x;
  const int per_xcd = nwg >> 3;
  const int logical = (bid & 7) * per_xcd + (bid >> 3);
  if (logical >= p.grid_real) return;
  // Items are (KV head, segment, row tile), row tiles innermost and the
  // longest causal rows first, so the XCDs of one KV head walk its K/V (L2
  // reuse).  When a KV head spans n_x whole XCDs its items are dealt to them
  // in turn (item i to XCD i mod n_x), so that every XCD gets long and short
  // rows alike and runs its longest first: a contiguous share would give one
  // XCD all the longest rows and end the launch late.
  const int per_g = p.splits * p.row_tiles;
  const int g = logical / per_g;
  int r = logical - g * per_g;
  if (per_g % per_xcd == 0) {
    const int n_x = per_g / per_xcd;
    r = (r % per_xcd) * n_x + r / per_xcd;
  }
  const int seg = r / p.row_tiles;
  const int rt = p.row_tiles - 1 - (r - seg * p.row_tiles);  // long rows first
  const int row0 = rt * kRowsPerWG;

  // This lane's rows, one per row block: query row `token` (head or tail
  // piece) at chunk position pos.
  auto chunk_pos = [&](int t) RA_INLINE {
    return t < p.head_rows ? p.head_pos + t : p.tail_pos + (t - p.head_rows);
  };
  int token[NRB], head[NRB], pos[NRB];
  bool row_ok[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = row0 + wave * kRowsPerWave + rb * 32 + lr;
    token[rb] = row / p.group;
    head[rb] = g * p.group + (row - token[rb] * p.group);
    pos[rb] = chunk_pos(token[rb]);
    row_ok[rb] = token[rb] < p.real_rows;
  }

  // Q^T operands: lane holds d = 16 s + 8 h + [0, 8) of each of its rows.
  // Loaded through a descriptor over this workgroup's tokens only (its base
  // at the first one, so offsets stay small at any q size), bounded at the
  // real rows: rows past them read 0.
  bf16x8 qreg[NRB][NKS];
  {
    const int t0 = row0 / p.group;
    const int t_end = min(p.real_rows, (row0 + kRowsPerWG - 1) / p.group + 1);
    const uint32_t q_bytes = t_end > t0 ? (uint32_t)(t_end - t0) * (uint32_t)p.nq * D * 2 : 0u;
    const __amdgpu_buffer_rsrc_t qr =
        make_rsrc(p.q + (int64_t)t0 * p.nq * D, q_bytes);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const uint32_t qoff = ((uint32_t)(token[rb] - t0) * p.nq + head[rb]) * D * 2 + 16 * h;
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        qreg[rb][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, qoff + 32 * s, 0, 0));
    }
  }

  // Tile schedule: ring region = P shard visits of nb tiles, then the
  // current tiles up to the largest chunk position among this workgroup's
  // real rows.  The rows [t0, t1] may straddle the head/tail boundary, so
  // the position range is taken over both pieces.
  const int t0 = row0 / p.group;
  const int t1 = min(p.real_rows - 1, (row0 + kRowsPerWG - 1) / p.group);
  int wg_min_pos, wg_max_pos;
  if (t1 < p.head_rows || t0 >= p.head_rows) {
    wg_min_pos = chunk_pos(t0);
    wg_max_pos = chunk_pos(t1);
  } else {
    wg_min_pos = min(chunk_pos(t0), p.tail_pos);
    wg_max_pos = max(chunk_pos(p.head_rows - 1), chunk_pos(t1));
  }
  // A partial launch walks one region only (its result is merged later).
  const int n_ring = (p.regions & 1) ? p.P * p.nb : 0;
  const int n_cur = (p.regions & 2) ? wg_max_pos / kBKV + 1 : 0;
  // This workgroup's segment of the walk: virtual tiles [v0, v0 + T).
  const int v0 = seg * p.seg_tiles;
  const int T = max(0, min(n_ring + n_cur - v0, p.seg_tiles));
  const uint32_t rowstride = (uint32_t)p.nkv * D * 2;  // bytes between tokens
  const uint32_t tile_stride = kBKV * rowstride;       // bytes between tiles
  // current tokens past the last position any row here sees load as zeros
  const uint32_t cur_bytes = (uint32_t)(wg_max_pos + 1) * rowstride;
  const int full_i = (int)p.full * p.interleave;  // < 2^31: bounded by a shard's length

  // The walk, one tile at a time from virtual tile v0: region k < P is the
  // visit of shard (ring_start - k) mod P (nb tiles), region P the current
  // tiles (n_cur), regions past it zero-size fetches (the slot fills with
  // zeros).  Three walkers hold one position of it each: the K copy two
  // tiles ahead, the V copy one tile ahead and the tile being computed
  // (its key bound).  A step adds to an offset and a bound; only entering
  // the next region, once per nb tiles, builds a descriptor.  The region's
  // descriptor is sized to its valid rows, so rows past them load as zeros.
  // Everything here is wave-uniform.
  struct Walker {
    i32x4 d;                // the region's K or V descriptor (base address, size in bytes)
    uint32_t off;           // byte offset of the tile's first row
    int lim;                // ring: valid keys of the visit left from this tile;
                            // current: chunk position of the tile's first key
    int left;               // tiles of the region from this one on
    int k;                  // region
    int dlim;               // lim's step per tile: -kBKV in a shard visit, +kBKV after
  };
  // enter region k at its tile b; side 0: K, 1: V
  auto enter = [&](Walker& w, int k, int b, int side) RA_INLINE {
    uint64_t base;
    uint32_t size;
    w.k = k;
    w.dlim = k < p.P ? -kBKV : kBKV;
    if (k < p.P) {
      int sh = p.ring_start - k;
      sh += (sh < 0) ? p.P : 0;
      const int len = full_i + min(max((int)p.rem - sh * p.interleave, 0), p.interleave);
      base = (uint64_t)(uintptr_t)(side ? p.v_cache : p.k_cache) +
             (uint64_t)(((int64_t)sh * p.shard_cap * p.nkv + g) * D) * 2u;
      size = (uint32_t)len * rowstride;
      w.lim = len - b * kBKV;
      w.left = p.nb - b;
    } else {
      base = (uint64_t)(uintptr_t)(side ? p.v_cur : p.k_cur) + (uint64_t)g * D * 2u;
      const bool cur = k == p.P && b < n_cur;
      size = cur ? cur_bytes : 0u;
      w.lim = b * kBKV;
      w.left = cur ? n_cur - b : (1 << 30);
    }
    w.d = make_desc(reinterpret_cast<const void*>(base), size);
    w.off = (uint32_t)b * tile_stride;
  };
  // one tile on; the region ends after `left` tiles
  auto step = [&](Walker& w, int side) RA_INLINE {
    w.off += tile_stride;
    w.lim += w.dlim;
    if (__builtin_expect(--w.left == 0, 0)) enter(w, w.k + 1, 0, side);
  };
  // the walkers at this workgroup's first tile
  Walker wk_, wv_, wb_;
  {
    int k0 = p.P, b0 = v0 - n_ring;
    if (n_ring == 0) {
      k0 = p.P;
    } else if (v0 < n_ring) {
      k0 = v0 / p.nb;
      b0 = v0 - k0 * p.nb;
    }
    enter(wk_, k0, b0, 0);
    enter(wv_, k0, b0, 1);
    wb_ = wk_;
  }
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
  auto desc_of = [](const Walker& w) RA_INLINE { return w.d; };
  auto issue_k = [&](const Walker& w, uint16_t* dst) RA_INLINE {
    const i32x4 d = desc_of(w);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int R = (wave * DPW + i) * RPI;
      dma16(d, dst + (wave * DPW + i) * 512, dma_kbase ^ (uint32_t)(swz_k(R, CPR) << 4),
            w.off + (uint32_t)R * rowstride);
    }
  };
  auto issue_v = [&](const Walker& w, uint16_t* dst) RA_INLINE {
    const i32x4 d = desc_of(w);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int R = (wave * DPW + i) * RPI;
      dma16(d, dst + (wave * DPW + i) * 512, dma_vbase ^ (uint32_t)(swz_v(R, CPR) << 4),
            w.off + (uint32_t)R * rowstride);
    }
  };
  // The copies issued from the hand-scheduled tile blocks split the rows
  // another way.  HD = 256: instruction 2 a + b of wave w moves rows R =
  // 2 w + 8 a + 16 b and R + 1; HD = 128 and 64: instruction b moves the
  // RPI rows from R = RPI w + 16 b on.  Rows 16 apart share their swizzle,
  // so one lane offset per operand and a (two at HD = 256) carries the
  // swizzle and R's rows for b = 0; the 16 more rows of b = 1 go into the
  // scalar offset (the sum, which the descriptor bounds, is the same).
  CopyLanes dl;
  const int dl_r0 = RPI * wave;  // the wave's first copied row
  {
    const int r0 = dl_r0, r1 = D == 256 ? dl_r0 + 8 : dl_r0;
    dl.ka = (dma_kbase ^ (uint32_t)(swz_k(r0, CPR) << 4)) + (uint32_t)r0 * rowstride;
    dl.kb = (dma_kbase ^ (uint32_t)(swz_k(r1, CPR) << 4)) + (uint32_t)r1 * rowstride;
    dl.va = (dma_vbase ^ (uint32_t)(swz_v(r0, CPR) << 4)) + (uint32_t)r0 * rowstride;
    dl.vb = (dma_vbase ^ (uint32_t)(swz_v(r1, CPR) << 4)) + (uint32_t)r1 * rowstride;
    dl.rs16 = 16 * rowstride;
  }
  const uint32_t m0b = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)dl_r0 * D * 2u);

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
  // Absolute LDS addresses for the hand-scheduled body: K reads ka[j] + slot,
  // V reads va[db % 4] + slot, the V slots counted from VBASE (d blocks 4..7
  // add 256: bit 8 of vbase is 0), so every offset stays below 64 KiB.
  uint32_t ka[8], va[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) ka[j] = lds0 + kx[j % NKX];
#pragma unroll
  for (int d = 0; d < 4; ++d) va[d] = lds0 + VBASE + (vbase ^ (uint32_t)(d << 6));

  f32x16 acc[NRB][NDB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[rb][db] = f32x16{};
  // bf16 probabilities of the previous tile (B operands of P.V); with fp32
  // output pb holds each probability's bf16 part and pbl the rest, rounded
  bf16x8 pb[NRB][NPS], pbl[NRB][NPS];
  // hand-scheduled blocks: bf16 output double-buffers the probabilities by
  // tile parity; fp32 output (HD = 256) keeps hi in pbuf[0] and lo in pbuf[1]
  bf16x8 pbuf[2][NRB][NPS];
  float mlog[NRB], lsum[NRB], lsum_q[NRB];  // running max (log2 units), row sums
  float lcomp[NRB], lcomp_q[NRB];            // their compensations (fold_sum)
  // hand-scheduled blocks: the row sums and compensations in two sets, read
  // by the softmax of even tiles from [0] (HD = 256; [1] in the three-tile
  // blocks) and of odd tiles from the other, each writing the set it does
  // not read; the final sums end in [0] either way
  float lsum2[2][NRB], lcomp2[2][NRB];
  // hand-scheduled blocks, bf16 output: the output's normaliser is lsum +
  // dq, dq the sum over significant tiles of (rounded - fp32) tile sums; a
  // tile is significant when a lane's tile sum exceeds its bound sbnd
  float dq[NRB], sbnd[NRB];
  // Three-tile blocks: the raw scores of the last two tiles, by tile parity.
  // Buffer 1 starts at -inf: the first block's softmax (of tile -1) then
  // yields zero probabilities.
  f32x16 sc[2][NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[0][rb][i] = 0.f;
      sc[1][rb][i] = kNegInf;
    }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    // a finite start (-FLT_MAX): the first max update needs no -inf guard,
    // and a row that never sees a key keeps l = 0 and gets lse = -inf
    mlog[rb] = -__FLT_MAX__;
    lsum[rb] = 0.f;     // fp32 sum of this lane's share of the keys' probabilities (LSE)
    lsum2[0][rb] = lcomp2[0][rb] = lsum2[1][rb] = lcomp2[1][rb] = 0.f;
    lsum_q[rb] = 0.f;   // the same over the bf16-rounded ones (generic bf16 normaliser)
    lcomp[rb] = lcomp_q[rb] = 0.f;
    dq[rb] = sbnd[rb] = 0.f;
  }
  const float c2 = p.scale_log2e;

  // S^T = K Q^T for one tile: every K operand read from LDS feeds the MFMAs
  // of all NRB row blocks.  Operands are read two k-steps ahead and the
  // schedule alternates one LDS read with the MFMAs of one step.
  auto qk = [&](const uint16_t* kt, f32x16 (&S)[NRB][NKB]) RA_INLINE {
    auto kop = [&](int s) RA_INLINE { return lds_read_b128(kt, kx[s & 7] + (s >> 3) * 256); };
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) S[rb][0] = f32x16{};
    bf16x8 kq[3];
    kq[0] = kop(0);
    kq[1] = kop(1);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      if (s + 2 < NKS) kq[(s + 2) % 3] = kop(s + 2);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        S[rb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[s % 3], qreg[rb][s], S[rb][0], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the first two LDS reads
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      if (s + 2 < NKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, NRB, 0);                 // NRB MFMAs
    }
  };

  // Region by value: keys with index >= lim[rb] in the tile are masked.
  // Lane half h holds keys (i / 4) * 8 + 4 h + i % 4 of each 32-key block,
  // so the compare is against the constant (i / 4) * 8 + i % 4.
  auto mask = [&](f32x16 (&S)[NRB][NKB], const int (&lim)[NRB]) RA_INLINE {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int l = lim[rb] - 4 * h;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          S[rb][kb][i] = kb * 32 + (i >> 2) * 8 + (i & 3) < l ? S[rb][kb][i] : kNegInf;
    }
  };

  // Probabilities -> bf16 B operands of P.V.  bf16 output: also the sum of
  // the bf16-rounded probabilities (v_dot2 against (1, 1)), the output's
  // normaliser, so numerator and denominator weight every key identically.
  // fp32 output: p = hi + lo, hi = bf16(p) and lo = bf16(p - hi), both
  // taken by P.V.
  auto pack = [&](const f32x16 (&S)[NRB][NKB], const float (&alpha)[NRB]) RA_INLINE {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float lq = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const bf16x2 pr = {(__bf16)S[rb][kb][i], (__bf16)S[rb][kb][i + 1]};
          if (!F32OUT) lq = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lq, false);
          pb[rb][2 * kb + (i >> 3)][i & 7] = pr[0];
          pb[rb][2 * kb + (i >> 3)][(i & 7) + 1] = pr[1];
          if (F32OUT) {
            pbl[rb][2 * kb + (i >> 3)][i & 7] = (__bf16)(S[rb][kb][i] - (float)pr[0]);
            pbl[rb][2 * kb + (i >> 3)][(i & 7) + 1] = (__bf16)(S[rb][kb][i + 1] - (float)pr[1]);
          }
        }
      if (!F32OUT) fold_sum(lsum_q[rb], lcomp_q[rb], alpha[rb], lq);
    }
  };

  // Region by value: each row's key bound within the tile, and whether any
  // bound of the workgroup cuts into the tile (then the compare is needed).
  auto bounds = [&](const Walker& w, int (&lim)[NRB]) RA_INLINE {
    const bool ring = w.k < p.P;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) lim[rb] = ring ? w.lim : pos[rb] + 1 - w.lim;
    return ring ? w.lim < kBKV : w.lim + kBKV > wg_min_pos + 1;
  };

  // P.V of the previous tile with the softmax of the current one (generic
  // head dims), hand ordered: slot t issues the MFMAs of P.V step t (one V
  // operand, read two slots ahead, for every row block) and then a fixed
  // slice of softmax work.  Softmax work units, in dependency order: the
  // in-lane max of each row block, the cross-lane reduction and new running
  // max, one exp2 per score, the row sums.  Returns the row blocks whose
  // rows must rescale the accumulator (al; 1 for the other rows).
  auto pv_softmax = [&](const uint16_t* vt, f32x16 (&S)[NRB][NKB], float (&al)[NRB]) RA_INLINE {
    constexpr int NT = NPS * NDB;                  // P.V steps
    constexpr int NE = NRB * NKB * 16;              // exp2 units
    constexpr int NU = NRB + 1 + NE + 1;            // all units
    auto vop = [&](int t) RA_INLINE {
      const int ks = t / NDB, db = t % NDB;
      const uint32_t o = (vbase ^ (uint32_t)(db << 6)) + ks * 16 * D * 2;
      const i16x4 x1 = lds_read_tr(vt, o);
      const i16x4 x2 = lds_read_tr(vt, o + 8 * D * 2);
      const i16x8 x = {x1[0], x1[1], x1[2], x1[3], x2[0], x2[1], x2[2], x2[3]};
      return __builtin_bit_cast(bf16x8, x);
    };
    float mx[NRB], m_use[NRB], ls[NRB];
    uint32_t any = 0;  // row blocks asking for a rescale
    auto unit = [&](int u) RA_INLINE {
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
          any |= anyrb ? 1u << rb : 0u;
        }
      } else if (u < NRB + 1 + NE) {  // one probability
        const int q = u - NRB - 1;
        const int rb = q / (NKB * 16), kb = (q / 16) % NKB, i = q % 16;
        S[rb][kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[rb][kb][i], c2, -m_use[rb]));
        ls[rb] += S[rb][kb][i];
      } else {  // row sums
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) fold_sum(lsum[rb], lcomp[rb], al[rb], ls[rb]);
      }
    };
    bf16x8 vq[3];
    vq[0] = vop(0);
    if (NT > 1) vq[1] = vop(1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int ks = t / NDB, db = t % NDB;
      if (t + 2 < NT) vq[(t + 2) % 3] = vop(t + 2);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        acc[rb][db] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[t % 3], pb[rb][ks], acc[rb][db], 0, 0, 0);
      if constexpr (F32OUT) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb)
          acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[t % 3], pbl[rb][ks],
                                                                acc[rb][db], 0, 0, 0);
      }
      // units [t*NU/NT, (t+1)*NU/NT), the rest after the last slot
#pragma unroll
      for (int u = t * NU / NT; u < (t + 1) * NU / NT; ++u) unit(u);
      __builtin_amdgcn_sched_barrier(0);
    }
    return any;
  };

  // Tiles run in pairs (2j, 2j+1); tile t's K and V live in slot t mod 4.
  // Tile t computes its scores from K(t), then issues its softmax between the
  // P.V MFMAs of tile t-1 (which read V(t-1)), then packs its probabilities;
  // the rare rescale for tile t's max is applied before the P.V of tile t.
  // At the start of pair j the copies for pair j+1 go out: K(2j+2), K(2j+3)
  // and, one tile behind, V(2j+1), V(2j+2); the slots they fill were last
  // read during pair j-1.  One wait and one barrier at the end of the pair
  // make them visible, so copies are in flight for a whole pair and the
  // workgroup synchronises every other tile.  Tiles at or past the end of
  // this workgroup's walk (t >= T) are fully masked: pass T carries the P.V
  // of the last tile.  Tile 0 runs the same body: its "previous" V slot is
  // filled with zeros and the probabilities start at zero.
  {
    Walker zero = wv_;
    zero.d[2] = 0;  // a zero-size fetch: the slot fills with zeros
    zero.off = 0;
    issue_k(wk_, kslot(0));
    step(wk_, 0);
    issue_k(wk_, kslot(1));
    step(wk_, 0);  // K copies run two tiles ahead ...
    if constexpr (ASMPIPE) {
      // ... and block u copies V tile u: tiles -2 and -1 (the P.V of the
      // first two blocks) read zeros
      issue_v(zero, vslot(2));
      issue_v(zero, vslot(3));
    } else {
      issue_v(zero, vslot(3));
      issue_v(wv_, vslot(0));
      step(wv_, 1);  // ... V copies one
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int ks = 0; ks < NPS; ++ks)
      pb[rb][ks] = pbl[rb][ks] = pbuf[0][rb][ks] = pbuf[1][rb][ks] = bf16x8{};
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
  __syncthreads();
  // Hand-scheduled blocks: the first two K operands of tile 0 (each block
  // reads them for the tile after it).
  bf16x8 kpre[2];
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (ASM256 || (ASMPIPE && D == 128))
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "={v[236:239]}"(kpre[0]), "={v[240:243]}"(kpre[1])
                 : "v"(ka[0]), "v"(ka[1])
                 : "memory");
#endif

  uint32_t resc = 0;      // row blocks whose rows the previous tile asked to rescale ...
  float alpha[NRB];       // ... by these factors (1 for the other rows)
  auto rescale = [&]() RA_INLINE {
    // (readfirstlane: resc is uniform, and so the test stays scalar)
    if (__builtin_expect(__builtin_amdgcn_readfirstlane(resc) != 0, 0)) {
#if defined(__HIP_DEVICE_COMPILE__)
      // the last P.V MFMAs may still be writing acc: wait them out
      asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
#endif
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
        if (resc & (1u << rb)) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) scale_agprs(acc[rb][db], alpha[rb]);
        }
    }
  };
  // Hand-scheduled blocks: the walkers' region changes and the key-bound
  // cuts happen at tiles known ahead, so the blocks keep two counters
  // instead of testing every tile.  cut_in: the tiles from the bound
  // walker's tile v on before the first one a key bound cuts -- in a shard
  // visit the one its keys end in (lim < 32), in the current tiles the first
  // whose first key passes the workgroup's smallest row position - 31 (from
  // there on every tile), and no later than the walk's end (every tile
  // past it is cut).  tn: the tiles before some walker enters its next
  // region; at 0 the walkers that finished theirs enter the next.
  auto cut_in = [&](const Walker& w, int v) RA_INLINE {
    int n = 0;  // past the regions every tile is cut
    if (w.k < p.P) {
      n = max(w.lim, 0) / kBKV;
    } else if (w.k == p.P) {
      const int d = wg_min_pos - 31 - w.lim;
      n = d < 0 ? 0 : d / kBKV + 1;
    }
    return min(n, T - v);
  };
  int nm = 0;                 // tiles before the next cut one (the blocks step it)
  uint32_t tn = 0, tn0 = 0;   // tiles before a region change; tn0: its value when set
  if constexpr (ASMBLK) {
    nm = cut_in(wb_, 0);
    tn = tn0 = (uint32_t)min(min(wb_.left, wk_.left), wv_.left);
  }
  auto region_change = [&](int v) RA_INLINE {  // after tile v: tn reached 0
    wb_.left -= (int)tn0;
    wk_.left -= (int)tn0;
    wv_.left -= (int)tn0;
    if (wb_.left == 0) {
      enter(wb_, wb_.k + 1, 0, 0);
      nm = cut_in(wb_, v + 1);
    }
    if (wk_.left == 0) enter(wk_, wk_.k + 1, 0, 0);
    if (wv_.left == 0) enter(wv_, wv_.k + 1, 0, 1);
    tn = tn0 = (uint32_t)min(min(wb_.left, wk_.left), wv_.left);
  };
  // Tile v, in slot SL = v mod 4.
  auto body = [&](auto slot, int v) RA_INLINE {
    constexpr int SL = decltype(slot)::value;
    rescale();
#ifdef RA_SYNC_EVERY_TILE  // checking build: every copy lands, every wave is here
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
#endif
    if constexpr (SL % 2 == 0 && !ASMBLK) {  // start of a pair: the copies of the next pair
      if (v + 2 <= T) {
        issue_k(wk_, kslot((SL + 2) % 4));
        step(wk_, 0);
        issue_k(wk_, kslot((SL + 3) % 4));
        step(wk_, 0);
        issue_v(wv_, vslot((SL + 1) % 4));
        step(wv_, 1);
        issue_v(wv_, vslot((SL + 2) % 4));
        step(wv_, 1);
      }
    }
    if constexpr (ASM256) {
      // a cut tile's key bound comes from these and the bound walker's lim
      // (on the mask's path); the block steps lim, the copy offsets and the
      // counters nm and tn
      const TileBound tb{wb_.k, p.P, v, T};

      // tile v's probabilities go to buffer v & 1; tile v-1's are read
      constexpr int PB = SL & 1;
      // this block's copies: K of tile v + 2 and V of tile v + 1
      const i32x4 dkr = desc_of(wk_), dvr = desc_of(wv_);
      tile_hd256<F32OUT, SL * TILE_B, ((SL + 3) % 4) * TILE_B, PB ^ 1, ((SL + 2) % 4) * TILE_B,
                 VBASE + ((SL + 1) % 4) * TILE_B, ((SL + 1) % 4) * TILE_B>(
          acc, pbuf[0], pbuf[1], qreg, kpre, ka, va, mlog, lsum2[SL & 1], lcomp2[SL & 1],
          lsum2[(SL & 1) ^ 1], lcomp2[(SL & 1) ^ 1], dq, sbnd, alpha, resc, c2, kTau<F32OUT>,
          kPBound, tb, pos, dkr, dvr, wk_.off, wv_.off, wb_.lim, wb_.dlim, nm, tn, tile_stride,
          m0b, dl);
      if (__builtin_expect(tn == 0, 0)) region_change(v);
    } else if constexpr (ASMPIPE) {
      // block v: scores of tile v, softmax of tile v-1, P.V of tile v-2
      const TileBound tb{wb_.k, p.P, v, T};
      // this block's copies: K of tile v + 2 and V of tile v
      const i32x4 dkr = desc_of(wk_), dvr = desc_of(wv_);
      tile_pipe<D, F32OUT, SL * TILE_B, ((SL + 2) % 4) * TILE_B, SL & 1,
                ((SL + 2) % 4) * TILE_B, VBASE + SL * TILE_B, ((SL + 1) % 4) * TILE_B>(
          acc, sc, pbuf[0], pbuf[1], qreg, kpre, ka, va, mlog, lsum2[SL & 1], lcomp2[SL & 1],
          lsum2[(SL & 1) ^ 1], lcomp2[(SL & 1) ^ 1], dq, sbnd, alpha, resc, c2, kTau<F32OUT>,
          kPBound, tb, pos, dkr, dvr, wk_.off, wv_.off, wb_.lim, wb_.dlim, nm, tn, tile_stride,
          m0b, dl);
      if (__builtin_expect(tn == 0, 0)) region_change(v);
    } else {
      int lim[NRB];
      bool cut = bounds(wb_, lim);
      step(wb_, 0);
      if (v >= T) {  // past the walk: every key masked
        cut = true;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) lim[rb] = -kBKV;
      }
      f32x16 S[NRB][NKB];
      qk(kslot(SL), S);
      if (cut) mask(S, lim);
      resc = pv_softmax(vslot((SL + 3) % 4), S, alpha);
      pack(S, alpha);
    }
#ifdef RA_SYNC_EVERY_TILE
    __syncthreads();
#endif
    if constexpr (SL % 2 == 1) {  // end of a pair
      if constexpr (!ASMBLK) {  // (the hand-scheduled blocks wait and synchronise themselves)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
        __syncthreads();
      }
    }
  };
  // Tiles 0 .. T (pass T is the P.V of the last tile; with the three-tile
  // blocks passes T and T + 1 are the softmax and the P.V of the last
  // tile), four per trip so that the slot offsets are constants.  The walk
  // ends on an odd pass, so the final row sums are in set 0.
  const int v_last = ASMPIPE ? T + 1 : T;
  for (int v = 0;;) {
    body(std::integral_constant<int, 0>{}, v);
    body(std::integral_constant<int, 1>{}, v + 1);
    if ((v += 2) > v_last) break;
    body(std::integral_constant<int, 2>{}, v);
    body(std::integral_constant<int, 3>{}, v + 1);
    if ((v += 2) > v_last) break;
  }

#if defined(__HIP_DEVICE_COMPILE__)
  // the last P.V MFMAs (inline asm, unseen by the compiler's hazard checks)
  // may still be writing acc, which is read below
  // (and the last block's KPRE reads may still be landing)
  if constexpr (ASMBLK) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#endif

  // Epilogue: out = acc / l, lse = ln 2 * (m + log2 l).  The lane's rows
  // are derived again here (lane id by mbcnt) rather than kept live through
  // the walk, where registers are scarce.
  const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int lr_e = lane_e & 31, h_e = lane_e >> 5;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = row0 + wave * kRowsPerWave + rb * 32 + lr_e;
    token[rb] = row / p.group;
    head[rb] = g * p.group + (row - token[rb] * p.group);
    row_ok[rb] = token[rb] < p.real_rows;
    // the LSE takes the fp32 sum; bf16 output is normalised by the sum of
    // the rounded probabilities its numerator took (hand-scheduled blocks:
    // of the significant tiles), fp32 output (hi + lo probabilities) by the
    // fp32 sum
    const float l_own = ASMBLK ? lsum2[0][rb] - lcomp2[0][rb] : lsum[rb] - lcomp[rb];
    const float lq_own = ASMBLK ? l_own + dq[rb] : lsum_q[rb] - lcomp_q[rb];
    const float l_tot = l_own + __shfl_xor(l_own, 32);
    const float l_norm = F32OUT ? l_tot : lq_own + __shfl_xor(lq_own, 32);
    if (!row_ok[rb]) continue;
    // a row that saw no key (possible in a one-region launch) gets out = 0
    // and lse = -inf (m = -inf, log2 0 = -inf)
    const float inv = l_norm > 0.f ? 1.f / l_norm : 0.f;
    // a split launch writes its segment's partial (out, lse)
    const int64_t obase = seg * p.seg_out_stride + ((int64_t)token[rb] * p.nq + head[rb]) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      if (F32OUT || p.store_f32) {
        // the two lane halves hold adjacent 4-value groups of a row: each
        // store writes 32 contiguous bytes per row
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int d0 = db * 32 + i4 * 8 + 4 * h_e;
          const f32x4 o = {acc[rb][db][4 * i4] * inv, acc[rb][db][4 * i4 + 1] * inv,
                           acc[rb][db][4 * i4 + 2] * inv, acc[rb][db][4 * i4 + 3] * inv};
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + obase + d0) = o;
        }
      } else {
        // bf16: groups i4 and i4 + 1 of both lane halves are exchanged
        // (v_permlane32_swap) so that the lower half holds values 0..7 of
        // group pair i4 and the upper half values 8..15: 16 bytes per lane,
        // 32 contiguous bytes per row and store
#pragma unroll
        for (int i4 = 0; i4 < 4; i4 += 2) {
          uint32_t a[2], b[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const bf16x2 pa = {(__bf16)(acc[rb][db][4 * i4 + 2 * k] * inv),
                               (__bf16)(acc[rb][db][4 * i4 + 2 * k + 1] * inv)};
            const bf16x2 pb = {(__bf16)(acc[rb][db][4 * i4 + 4 + 2 * k] * inv),
                               (__bf16)(acc[rb][db][4 * i4 + 4 + 2 * k + 1] * inv)};
            a[k] = __builtin_bit_cast(uint32_t, pa);
            b[k] = __builtin_bit_cast(uint32_t, pb);
          }
          const auto s0 = __builtin_amdgcn_permlane32_swap(a[0], b[0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(a[1], b[1], false, false);
          const int d0 = db * 32 + (i4 + h_e) * 8;
          const i32x4 v = {(int)s0[0], (int)s1[0], (int)s0[1], (int)s1[1]};
          *reinterpret_cast<i32x4*>(static_cast<uint16_t*>(p.out) + obase + d0) = v;
        }
      }
    }
    if (h_e == 0 && p.lse != nullptr)
      p.lse[((int64_t)seg * p.nq + head[rb]) * p.q_rows + token[rb]] =
          (mlog[rb] + __log2f(l_tot)) * kLn2;
  }

  // The fused strided write: this workgroup's tokens of the chunk go to their
  // cache slots (position p = write_pos0 + t: shard (p / I) mod P, slot
  // ((p / I) / P) * I + p mod I), 16 bytes a thread, K and V alike.  The
  // walk reads positions below write_pos0 only, so no workgroup reads a slot
  // written here.
  if (p.write_tokens > 0) {
    const int64_t t0 = (int64_t)logical * p.write_per_wg;
    const int64_t t1 = min((int64_t)p.write_tokens, t0 + p.write_per_wg);
    // the thread's index from the wave id (an SGPR) and the lane id, as in
    // the epilogue: keeping threadIdx.x in a VGPR across the walk would
    // spill it
    const int tid_w = wave * 64 + lane_e;
    for (int64_t idx = t0 * p.write_chunks + tid_w; idx < t1 * p.write_chunks;
         idx += kWaves * 64) {
      const int64_t t = idx / p.write_chunks;
      const int c = (int)(idx - t * p.write_chunks);
      const int64_t pos = p.write_pos0 + t;
      const int64_t unit = pos / p.interleave;
      const int64_t sh = unit % p.P;
      const int64_t slot = (unit / p.P) * p.interleave + (pos - unit * p.interleave);
      const int64_t dst = (sh * p.shard_cap + slot) * p.write_chunks + c;
      const i32x4 kx = reinterpret_cast<const i32x4*>(p.k_cur)[idx];
      const i32x4 vx = reinterpret_cast<const i32x4*>(p.v_cur)[idx];
      reinterpret_cast<i32x4*>(p.wk_cache)[dst] = kx;
      reinterpret_cast<i32x4*>(p.wv_cache)[dst] = vx;
    }
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
