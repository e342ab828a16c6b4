/*
 * libringattn -- fused ring + current causal attention for chunked prefill,
 * and the strided KV-cache write that fills its striped cache (MI355X, gfx950).
 *
 * Source of the method: vLLM tpu-inference pull request "PCP: in-kernel ring
 * cache phase, fused with the current phase".
 *   - Summary: the ring cache rounds and the causal current phase run in ONE
 *     launch sharing one online softmax; no second launch, no LSE merge.
 *   - Design: per query block the key walk visits the ring region (the P
 *     striped cache shards) and then the current-KV blocks (causal); region
 *     behaviour is selected by value; current KV is passed in token order.
 *   - Testing: ring agrees with attention over the gathered cache; the
 *     strided KV-cache write is bit-exact.
 * On one GPU the ring hops between ranks become sequential shard visits
 * inside the kernel; a call computes one rank's share at its real shape.
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers owned by the caller, dense
 *     row-major, 16-byte aligned.  bf16 is IEEE bfloat16 (1-8-7).
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *     the default stream).  They do not synchronise the host, allocate, or
 *     copy host to device, and keep no pointer after returning; buffers must
 *     stay alive until the stream has run the work.  A call puts only kernel
 *     launches on the stream (no memset, no copy), so it may be captured into
 *     a HIP graph, which reads the buffers at each replay.  Apart from
 *     ring_attn_prefill_split_noalloc, calls share no device state, and
 *     calls on different streams may run concurrently.
 *   - Every argument is validated on the host before any HIP call.  On error
 *     nothing is launched, a non-zero ra_status_t is returned and
 *     ra_last_error() describes it.  Launch failures return RA_ERR_HIP.
 *
 * Striped cache ("striped shard", Design section).  Cached token positions
 * are dealt to shards 0..P-1 in turn, in units of `interleave` consecutive
 * tokens (interleave = 1: token round-robin).  Position p lives in
 *     shard = (p / I) mod P,   slot = ((p / I) / P) * I + p mod I.
 * A cache holding positions [0, cache_len) gives shard s the length
 *     full*I + clamp(rem - s*I, 0, I),  full = cache_len / (P*I),
 *                                        rem  = cache_len mod (P*I).
 * Cache tensors are laid out [P, shard_cap, NKV, HD]; slots at or beyond a
 * shard's length are never read (they may hold anything, NaN included).
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_INVALID_ARG = 1, /* argument out of its documented domain */
  RA_ERR_UNSUPPORTED = 2, /* valid, but outside what this build implements */
  RA_ERR_HIP = 3          /* the HIP runtime refused the launch */
} ra_status_t;

typedef enum { RA_DTYPE_BF16 = 0, RA_DTYPE_FP32 = 1 } ra_dtype_t;

/* Key regions of one launch (ring_attn_partial). */
typedef enum {
  RA_REGION_CACHE = 1,  /* the P cache shards (ring rounds) */
  RA_REGION_CURRENT = 2 /* the causal current chunk */
} ra_region_t;

/* Stripe layout of the cache.  ring_start is the first shard visited; the
 * visit order is ring_start, ring_start-1, ... (mod P), the order in which a
 * rank sees its neighbours' shards arrive.  The result does not depend on it
 * beyond floating-point rounding order. */
typedef struct {
  int32_t interleave; /* tokens per stripe unit, >= 1 */
  int32_t ring_start; /* in [0, P) */
} ra_stripe_layout_t;

/* Shapes.  The query rows are a head piece of head_rows rows followed by a
 * tail piece of q_rows - head_rows rows (Design section: the current phase
 * keeps its two-sequence (head, tail) structure, both padded to full
 * length, and the caller discards pad rows).  The pieces sit at chunk
 * positions head_pos and tail_pos: query row i is the token at chunk
 * position
 *     pos(i) = head_pos + i                for i <  head_rows,
 *              tail_pos + (i - head_rows)  for i >= head_rows,
 * i.e. at global position cache_len + pos(i), and it sees current tokens
 * 0..pos(i).  The contiguous layout is head_pos = 0, tail_pos = head_rows;
 * the load-balanced context-parallel layout gives rank r of R the pieces r
 * and 2R-1-r of a chunk cut into 2R.  The current K/V hold cur_len tokens
 * of the chunk in token order (Design, first subtlety).  Rows [0, real_rows)
 * are real; rows [real_rows, q_rows) are pads: their out/lse entries are
 * not written, and current tokens past the last real row's position are
 * never read as keys. */
typedef struct {
  int32_t num_q_heads;  /* NQ >= 1 */
  int32_t num_kv_heads; /* NKV >= 1, NQ % NKV == 0; query head h reads KV
                           head h / (NQ / NKV) */
  int32_t head_dim;     /* HD in {64, 128, 256} */
  int32_t q_rows;       /* C >= 0 */
  int32_t head_rows;    /* 0 <= head_rows <= q_rows */
  int32_t real_rows;    /* 0 <= real_rows <= q_rows */
  int32_t head_pos;     /* chunk position of query row 0, >= 0 */
  int32_t tail_pos;     /* chunk position of query row head_rows, >= 0 */
  int32_t cur_len;      /* tokens in k_cur / v_cur; every real row's
                           position must be < cur_len */
  int64_t shard_cap;    /* slots allocated per shard, >= 1 */
  float scale;          /* softmax scale, finite and > 0; 0 selects
                           1/sqrt(HD); negative scales are rejected */
  int32_t out_dtype;    /* ra_dtype_t of `out` */
} ra_dims_t;

/*
 * ring_attn_prefill -- one launch: all P shard visits, then the causal
 * current chunk, through one online softmax (Summary and Design sections).
 *
 *   q        bf16 [C, NQ, HD]             chunk queries
 *   k_cache  bf16 [P, shard_cap, NKV, HD] striped cache keys (read only)
 *   v_cache  bf16 [P, shard_cap, NKV, HD] striped cache values (read only)
 *   k_cur    bf16 [cur_len, NKV, HD]  current keys, TOKEN order: row j is
 *                               global position cache_len + j
 *   v_cur    bf16 [cur_len, NKV, HD]  current values, token order
 *   cache_len  number of cached positions, >= 0 (0: no ring region)
 *   P          number of shards, >= 1
 *   out      [C, NQ, HD] bf16 or fp32 (dims->out_dtype); real row i gets
 *            softmax(scale * q k^T) v over cache positions [0, cache_len)
 *            and current tokens 0..pos(i)
 *   lse      fp32 [NQ, C] natural-log log-sum-exp of the scaled scores of
 *            each real row, or NULL to skip
 *
 * k_cache/v_cache may be NULL only when cache_len == 0.  out and lse must
 * not overlap any input.  Limits (RA_ERR_UNSUPPORTED beyond them): each
 * shard's valid rows plus one 32-key tile, and cur_len plus one tile, stay
 * below 2^31 bytes of K (NKV * HD * 2 bytes a row); (256 / (NQ/NKV) + 2) *
 * NQ * HD * 2 < 2^31 (the q rows one workgroup reads); real_rows * NQ/NKV
 * < 2^30.  q, out and the caches may be larger than 4 GiB.
 * Returns RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED or RA_ERR_HIP.
 */
int ring_attn_prefill(const void* q, const void* k_cache, const void* v_cache,
                      const void* k_cur, const void* v_cur, int64_t cache_len,
                      int32_t P, ra_stripe_layout_t stripe_layout, void* out,
                      float* lse, const ra_dims_t* dims, void* stream);

/*
 * ring_attn_prefill_write -- ring_attn_prefill and kv_cache_write of the
 * same chunk in one launch: the pages pair the fused attention launch with
 * a strided write of the chunk's K/V into the striped cache (Summary
 * section; Testing section: the write is bit-exact).  Arguments as
 * ring_attn_prefill, the caches writable, plus
 *   n_tokens  current tokens 0 .. n_tokens-1 to write, 0 <= n_tokens <=
 *             dims->cur_len; token t goes to global position cache_len + t
 *             exactly as kv_cache_write puts it
 * The walk reads cache positions below cache_len only and the write touches
 * positions from cache_len on, so out, lse and the caches equal those of
 * kv_cache_write and ring_attn_prefill called one after the other, bit for
 * bit.  Every written slot must be < shard_cap; the caches must not overlap
 * q, k_cur, v_cur, out or lse, nor each other (RA_ERR_INVALID_ARG).  One
 * launch, never split.  With real_rows == 0 only the write runs; with
 * n_tokens == 0 only the attention.
 */
int ring_attn_prefill_write(const void* q, void* k_cache, void* v_cache, const void* k_cur,
                            const void* v_cur, int64_t cache_len, int32_t P,
                            ra_stripe_layout_t stripe_layout, int32_t n_tokens, void* out,
                            float* lse, const ra_dims_t* dims, void* stream);

/* Largest number of segments a split launch may cut each row's walk into. */
#define RA_MAX_SPLITS 64

/*
 * ring_attn_prefill_split -- ring_attn_prefill with the key walk of every
 * row cut into `splits` consecutive segments (in walk order: shard visits,
 * then current blocks) run by separate workgroups.  Each segment's
 * (m, l, acc) is spilled to `workspace` as a normalised partial output and
 * its LSE, and one log-sum-exp merge forms out and lse.  The pages name an
 * HBM-spilled (m, l, acc) as the follow-up for long contexts (Performance
 * section); on one GPU the split serves parallelism: a rank's share of a few
 * hundred rows fills only a fraction of the chip unless its walk is split.
 * Same arguments and result as ring_attn_prefill, plus
 *   splits           1 .. RA_MAX_SPLITS (1: ring_attn_prefill itself)
 *   workspace        caller-owned device scratch, 16-byte aligned, at least
 *                    ra_split_workspace_bytes() bytes; overwritten; must not
 *                    overlap any tensor argument; unused when splits == 1
 *   workspace_bytes  its size
 * The partials are fp32 whatever the output dtype, so the result is rounded
 * once, after the merge.
 */
int ring_attn_prefill_split(const void* q, const void* k_cache, const void* v_cache,
                            const void* k_cur, const void* v_cur, int64_t cache_len,
                            int32_t P, ra_stripe_layout_t stripe_layout, int32_t splits,
                            void* workspace, int64_t workspace_bytes, void* out, float* lse,
                            const ra_dims_t* dims, void* stream);

/*
 * ring_attn_prefill_split_write -- ring_attn_prefill_split with the
 * strided cache write of ring_attn_prefill_write in the same launch (the
 * split walk's segments share the copy of the chunk's tokens); the merge
 * follows as its own launch.  Arguments: those of ring_attn_prefill_split,
 * the caches writable, plus n_tokens as in ring_attn_prefill_write, whose
 * checks also apply (the workspace must not overlap the caches either).
 * splits == 1 is ring_attn_prefill_write.  Result: that of kv_cache_write
 * followed by ring_attn_prefill_split, bit for bit.
 */
int ring_attn_prefill_split_write(const void* q, void* k_cache, void* v_cache, const void* k_cur,
                                  const void* v_cur, int64_t cache_len, int32_t P,
                                  ra_stripe_layout_t stripe_layout, int32_t splits,
                                  void* workspace, int64_t workspace_bytes, int32_t n_tokens,
                                  void* out, float* lse, const ra_dims_t* dims, void* stream);

/* Bytes of the workspace ring_attn_prefill_split_noalloc keeps in the
 * library's own device memory (one copy per GPU, held until the process
 * ends): 72 MiB, e.g. splits = 4 over a 512-row rank share at NQ = 32,
 * HD = 256. */
#define RA_NOALLOC_SCRATCH_BYTES (72ll << 20)

/*
 * ring_attn_prefill_split_noalloc -- ring_attn_prefill_split without a
 * caller workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The segments' partials go to a workspace of
 * RA_NOALLOC_SCRATCH_BYTES that the library holds per GPU; the call itself
 * allocates nothing.  Same arguments and result as ring_attn_prefill_split
 * minus workspace / workspace_bytes.  The stream must belong to the
 * current device (hipSetDevice); the first call on a device looks the
 * workspace up there.
 *
 * Every call on one GPU shares that GPU's workspace, and the workspace
 * keeps the last call's contents (every partial a call reads is written by
 * the same call first, so nothing needs clearing).  Calls that overlap on
 * one GPU -- on different streams, or in parallel host threads -- race on
 * it: order them on one stream.
 *
 * Returns RA_ERR_UNSUPPORTED (nothing launched) when splits > 1 needs more
 * than RA_NOALLOC_SCRATCH_BYTES (see ra_split_workspace_bytes), else as
 * ring_attn_prefill_split.
 */
int ring_attn_prefill_split_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const void* k_cur, const void* v_cur, int64_t cache_len,
                                    int32_t P, ra_stripe_layout_t stripe_layout, int32_t splits,
                                    void* out, float* lse, const ra_dims_t* dims, void* stream);

/* Host-only: a split count for these dims on a GPU with num_cus compute
 * units.  One workgroup (256 query rows of one KV head) runs per CU at a
 * time (two at HD = 64); the count is chosen so that the workgroups of all segments fill the
 * last wave best, charging each extra segment a small cost (1: no split).
 * Writes *splits; no GPU involved. */
int ra_split_suggest(const ra_dims_t* dims, int32_t num_cus, int32_t* splits);

/* Host-only: workspace bytes ring_attn_prefill_split needs for these dims and
 * splits (0 when splits == 1).  Writes *bytes; no GPU involved. */
int ra_split_workspace_bytes(const ra_dims_t* dims, int32_t splits, int64_t* bytes);

/*
 * ring_attn_partial -- the same launch restricted to some key regions:
 * regions = RA_REGION_CACHE (the cache-only ring launch), RA_REGION_CURRENT
 * (the causal current phase alone) or both (= ring_attn_prefill).  The
 * Summary section describes the removed two-launch variant (a cache-only
 * ring launch plus an LSE merge); these calls and merge_attn_states rebuild
 * it as the fused launch's comparator.  Arguments as ring_attn_prefill; a
 * real row that sees no key in the chosen regions (a cache-only launch with
 * cache_len == 0) gets out = 0 and lse = -inf.  For merging, keep the LSE.
 */
int ring_attn_partial(const void* q, const void* k_cache, const void* v_cache,
                      const void* k_cur, const void* v_cur, int64_t cache_len,
                      int32_t P, ra_stripe_layout_t stripe_layout, int32_t regions,
                      void* out, float* lse, const ra_dims_t* dims, void* stream);

/*
 * merge_attn_states -- log-sum-exp merge of two partial attentions of the
 * same rows over disjoint key sets (the merge of the removed two-launch
 * variant, Summary section).  For every real row and query head:
 *     lse = log(exp(lse1) + exp(lse2)),
 *     out = exp(lse1 - lse) * o1 + exp(lse2 - lse) * o2,
 * a part with lse = -inf weighted 0; out = 0 and lse = -inf when both are.
 *
 *   o1, o2      [C, NQ, HD] partial outputs, bf16 or fp32 (parts_dtype)
 *   lse1, lse2  fp32 [NQ, C]       their natural-log LSEs
 *   parts_dtype ra_dtype_t of o1 and o2 (the merge itself runs in fp32)
 *   out         [C, NQ, HD] bf16 or fp32 (dims->out_dtype)
 *   lse         fp32 [NQ, C] merged LSE, or NULL to skip
 *   dims        uses num_q_heads, head_dim, q_rows, real_rows, out_dtype
 *
 * Pad rows (>= real_rows) are not written.  out and lse must not overlap an
 * input.  Returns RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED or
 * RA_ERR_HIP.
 */
int merge_attn_states(const void* o1, const float* lse1, const void* o2, const float* lse2,
                      int32_t parts_dtype, void* out, float* lse, const ra_dims_t* dims,
                      void* stream);

/*
 * kv_cache_write -- strided write of the chunk's current K/V into the
 * striped cache (Design section: striped shards; Testing section: the write
 * is bit-exact).  Current token t < n_tokens (global position
 * cache_len + t) is copied bit for bit to its (shard, slot) in k_cache and
 * v_cache.  No other slot is touched.  It only writes slots that
 * ring_attn_prefill with the same cache_len never reads, so the two calls
 * commute.
 *
 *   k_cur, v_cur      bf16 [>= n_tokens, NKV, HD], token order
 *   n_tokens          real tokens to write, >= 0 (pads are not written)
 *   k_cache, v_cache  bf16 [P, shard_cap, NKV, HD]
 *   dims              uses num_kv_heads, head_dim, shard_cap only
 *
 * Every written slot must be < shard_cap (else RA_ERR_INVALID_ARG).
 */
int kv_cache_write(const void* k_cur, const void* v_cur, int32_t n_tokens,
                   void* k_cache, void* v_cache, int64_t cache_len, int32_t P,
                   ra_stripe_layout_t stripe_layout, const ra_dims_t* dims,
                   void* stream);

/* Host-only: length of shard `shard` when positions [0, cache_len) are
 * cached, by the closed form above.  Writes *len; no GPU involved. */
int ra_shard_len(int64_t cache_len, int32_t P, ra_stripe_layout_t stripe_layout,
                 int32_t shard, int64_t* len);

/* Thread-local text for the last non-OK status returned on this thread. */
const char* ra_last_error(void);

/* Library version string. */
const char* ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RINGATTN_H */
