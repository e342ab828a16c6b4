// C entry points of libringattn: argument validation, stripe geometry and
// kernel dispatch.  Everything here runs on the host; the only HIP calls
// are the asynchronous launches, made after every check has passed.
//
// Stripe geometry follows the vLLM tpu-inference pull request "PCP: in-kernel
// ring cache phase, fused with the current phase", Design section (striped
// cache shards visited as ring rounds, the cache bound of a partial last
// block applied at run time).
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/ringattn.h"
#include "ra_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + na) and [b, b + nb) overlap (byte ranges; empty ranges never do).
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Length of shard s when positions [0, cache_len) are cached (closed form of
// the round-robin deal in units of `interleave` tokens).
int64_t shard_len(int64_t cache_len, int32_t P, int32_t interleave, int32_t s) {
  const int64_t round = (int64_t)P * interleave;
  const int64_t full = cache_len / round, rem = cache_len % round;
  int64_t extra = rem - (int64_t)s * interleave;
  extra = extra < 0 ? 0 : (extra > interleave ? interleave : extra);
  return full * interleave + extra;
}

int check_layout(int32_t P, ra_stripe_layout_t s, int64_t cache_len) {
  if (P < 1) return fail(RA_ERR_INVALID_ARG, "P must be >= 1; got %d", P);
  if (s.interleave < 1)
    return fail(RA_ERR_INVALID_ARG, "stripe_layout.interleave must be >= 1; got %d", s.interleave);
  if (s.ring_start < 0 || s.ring_start >= P)
    return fail(RA_ERR_INVALID_ARG, "stripe_layout.ring_start must be in [0, P=%d); got %d", P,
                s.ring_start);
  if (cache_len < 0) return fail(RA_ERR_INVALID_ARG, "cache_len must be >= 0; got %lld",
                                 (long long)cache_len);
  return RA_OK;
}

int check_heads(const ra_dims_t* d) {
  if (!d) return fail(RA_ERR_INVALID_ARG, "dims must not be NULL");
  if (d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(RA_ERR_INVALID_ARG, "num_q_heads (%d) and num_kv_heads (%d) must be >= 1",
                d->num_q_heads, d->num_kv_heads);
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(RA_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                d->num_q_heads, d->num_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
    return fail(RA_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256; got %d", d->head_dim);
  if (d->shard_cap < 1)
    return fail(RA_ERR_INVALID_ARG, "shard_cap must be >= 1; got %lld", (long long)d->shard_cap);
  return RA_OK;
}

}  // namespace

extern "C" {

const char* ra_last_error(void) { return g_last_error.c_str(); }

const char* ra_version(void) {
#ifdef RA_SYNC_EVERY_TILE
  return "libringattn 0.1 (gfx950, checking build: synchronised every tile)";
#else
  return "libringattn 0.1 (gfx950)";
#endif
}

int ra_shard_len(int64_t cache_len, int32_t P, ra_stripe_layout_t stripe_layout, int32_t shard,
                 int64_t* len) {
  if (int rc = check_layout(P, stripe_layout, cache_len)) return rc;
  if (shard < 0 || shard >= P)
    return fail(RA_ERR_INVALID_ARG, "shard must be in [0, P=%d); got %d", P, shard);
  if (!len) return fail(RA_ERR_INVALID_ARG, "len must not be NULL");
  *len = shard_len(cache_len, P, stripe_layout.interleave, shard);
  return RA_OK;
}

}  // extern "C"

namespace {

// Bytes of a split launch's workspace: the partial outputs [S, C, NQ, HD]
// fp32 (a bf16 partial would round twice, once there and once after the
// merge) then the partial LSEs [S, NQ, C] fp32, both 256-byte aligned.
int64_t split_part_bytes(const ra_dims_t& d, int32_t splits) {
  const int64_t o = (int64_t)splits * d.q_rows * d.num_q_heads * d.head_dim * 4;
  return (o + 255) / 256 * 256;
}
int64_t split_workspace_bytes(const ra_dims_t& d, int32_t splits) {
  const int64_t l = (int64_t)splits * d.num_q_heads * d.q_rows * 4;
  return split_part_bytes(d, splits) + (l + 255) / 256 * 256;
}

// With RINGATTN_LOG=1 in the environment, the first fused launch of the
// process prints its geometry to stderr (once; later launches are silent).
void log_geometry(const ra::FusedParams& p, int hd) {
  static std::atomic<bool> done{false};
  const char* v = std::getenv("RINGATTN_LOG");
  if (!v || std::strcmp(v, "1") != 0 || done.exchange(true)) return;
  std::fprintf(stderr,
               "libringattn: fused launch HD=%d NQ=%d NKV=%d rows=%d (real %d, head %d at %d, "
               "tail at %d) P=%d I=%d ring_start=%d full=%lld rem=%lld tiles/visit=%d "
               "row_tiles=%d splits=%d seg_tiles=%d regions=%d workgroups=%d (+%d padding) "
               "x %d threads, out %s\n",
               hd, p.nq, p.nkv, p.q_rows, p.real_rows, p.head_rows, p.head_pos, p.tail_pos, p.P,
               p.interleave, p.ring_start, (long long)p.full, (long long)p.rem, p.nb,
               p.row_tiles, p.splits, p.seg_tiles, p.regions, p.grid_real,
               (p.grid_real + 7) / 8 * 8 - p.grid_real, ra::kWaves * 64,
               p.out_f32 ? "fp32" : "bf16");
}

// ring_attn_prefill over the regions selected by `regions` (1: cache, 2:
// current, 3: both), with the walk of every row tile cut into `splits`
// segments.  With splits > 1, out and lse receive the segments' partials
// ([splits, C, NQ, HD] and [splits, NQ, C]).
// The strided cache write a launch may carry (ring_attn_prefill_write).
struct FusedWrite {
  void* k_cache;
  void* v_cache;
  int32_t n_tokens;
};

int prefill_regions(const void* q, const void* k_cache, const void* v_cache, const void* k_cur,
                    const void* v_cur, int64_t cache_len, int32_t P,
                    ra_stripe_layout_t stripe_layout, int32_t regions, void* out, float* lse,
                    const ra_dims_t* dims, void* stream, int32_t splits = 1,
                    const FusedWrite* write = nullptr) {
  if (int rc = check_heads(dims)) return rc;
  if (int rc = check_layout(P, stripe_layout, cache_len)) return rc;
  const ra_dims_t& d = *dims;
  const int32_t C = d.q_rows;
  if (C < 0) return fail(RA_ERR_INVALID_ARG, "q_rows must be >= 0; got %d", C);
  if (d.head_rows < 0 || d.head_rows > C)
    return fail(RA_ERR_INVALID_ARG, "head_rows must be in [0, q_rows=%d]; got %d", C, d.head_rows);
  if (d.real_rows < 0 || d.real_rows > C)
    return fail(RA_ERR_INVALID_ARG, "real_rows must be in [0, q_rows=%d]; got %d", C, d.real_rows);
  if (d.head_pos < 0 || d.tail_pos < 0 || d.cur_len < 0)
    return fail(RA_ERR_INVALID_ARG, "head_pos (%d), tail_pos (%d) and cur_len (%d) must be >= 0",
                d.head_pos, d.tail_pos, d.cur_len);
  // The largest chunk position among the real rows (-1 when there are none).
  int64_t max_pos = -1;
  if (d.real_rows > 0) {
    const int32_t real_head = d.real_rows < d.head_rows ? d.real_rows : d.head_rows;
    if (real_head > 0) max_pos = (int64_t)d.head_pos + real_head - 1;
    if (d.real_rows > d.head_rows) {
      const int64_t t = (int64_t)d.tail_pos + (d.real_rows - d.head_rows) - 1;
      max_pos = t > max_pos ? t : max_pos;
    }
  }
  if (max_pos >= d.cur_len)
    return fail(RA_ERR_INVALID_ARG,
                "real rows reach chunk position %lld but k_cur/v_cur hold cur_len=%d tokens",
                (long long)max_pos, d.cur_len);
  if (d.out_dtype != RA_DTYPE_BF16 && d.out_dtype != RA_DTYPE_FP32)
    return fail(RA_ERR_INVALID_ARG, "out_dtype must be RA_DTYPE_BF16 or RA_DTYPE_FP32; got %d",
                d.out_dtype);
  if (!std::isfinite(d.scale) || d.scale < 0.f)
    return fail(RA_ERR_INVALID_ARG,
                "scale must be finite and >= 0 (0 selects 1/sqrt(head_dim)); got %g",
                (double)d.scale);
  const int32_t NQ = d.num_q_heads, NKV = d.num_kv_heads, HD = d.head_dim;
  const int32_t group = NQ / NKV;

  // Shards: the first shard is the longest.
  const int64_t max_len = shard_len(cache_len, P, stripe_layout.interleave, 0);
  if (max_len > d.shard_cap)
    return fail(RA_ERR_INVALID_ARG,
                "cache_len %lld needs %lld slots in shard 0 but shard_cap is %lld",
                (long long)cache_len, (long long)max_len, (long long)d.shard_cap);

  if (d.real_rows == 0) return RA_OK;  // nothing real to compute

  if (!q || !k_cur || !v_cur || !out)
    return fail(RA_ERR_INVALID_ARG, "q, k_cur, v_cur and out must not be NULL");
  if (cache_len > 0 && (!k_cache || !v_cache))
    return fail(RA_ERR_INVALID_ARG, "k_cache and v_cache must not be NULL when cache_len > 0");
  const void* ptrs[] = {q, k_cache, v_cache, k_cur, v_cur, out, lse};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr))
      return fail(RA_ERR_INVALID_ARG, "every tensor pointer must be 16-byte aligned");

  // 32-bit buffer offsets: a shard visit reads at most max_len + BKV rows,
  // the current region at most cur_len + BKV rows.
  const int64_t rowstride = (int64_t)NKV * HD * 2;
  const int64_t lim31 = (int64_t)1 << 31;
  if ((max_len + ra::kBKV) * rowstride >= lim31)
    return fail(RA_ERR_UNSUPPORTED, "a shard of %lld tokens x %lld bytes exceeds 2 GiB",
                (long long)max_len, (long long)rowstride);
  if (((int64_t)d.cur_len + ra::kBKV) * rowstride >= lim31)
    return fail(RA_ERR_UNSUPPORTED, "the current chunk (%d tokens x %lld bytes) exceeds 2 GiB",
                d.cur_len, (long long)rowstride);
  // Each workgroup reads its own tokens' q rows through one descriptor.
  if ((int64_t)(ra::kRowsPerWG / group + 2) * NQ * HD * 2 >= lim31)
    return fail(RA_ERR_UNSUPPORTED, "num_q_heads=%d with %d q heads per KV head is too large",
                NQ, group);
  const int64_t rows_total = (int64_t)d.real_rows * group;
  if (rows_total + ra::kRowsPerWG >= lim31 / 2)
    return fail(RA_ERR_UNSUPPORTED, "real_rows * (NQ/NKV) = %lld is too large",
                (long long)rows_total);

  // Outputs must not alias inputs.
  const int64_t q_bytes = (int64_t)C * NQ * HD * 2;
  const int64_t cur_bytes = (int64_t)d.cur_len * NKV * HD * 2;
  const int64_t cache_bytes = (int64_t)P * d.shard_cap * NKV * HD * 2;
  // a split launch writes fp32 partials ([splits, C, NQ, HD])
  const int64_t out_bytes =
      (int64_t)splits * C * NQ * HD * (d.out_dtype == RA_DTYPE_FP32 || splits > 1 ? 4 : 2);
  const int64_t lse_bytes = (int64_t)splits * NQ * C * 4;
  struct R { const void* p; int64_t n; };
  const R ins[] = {{q, q_bytes}, {k_cache, cache_len > 0 ? cache_bytes : 0},
                   {v_cache, cache_len > 0 ? cache_bytes : 0}, {k_cur, cur_bytes},
                   {v_cur, cur_bytes}};
  for (const R& r : ins) {
    if (overlaps(out, out_bytes, r.p, r.n))
      return fail(RA_ERR_INVALID_ARG, "out overlaps an input tensor");
    if (overlaps(lse, lse_bytes, r.p, r.n))
      return fail(RA_ERR_INVALID_ARG, "lse overlaps an input tensor");
  }
  if (overlaps(out, out_bytes, lse, lse_bytes))
    return fail(RA_ERR_INVALID_ARG, "out and lse overlap");

  ra::FusedParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.k_cur = static_cast<const uint16_t*>(k_cur);
  p.v_cur = static_cast<const uint16_t*>(v_cur);
  p.out = out;
  p.lse = lse;
  p.shard_cap = d.shard_cap;
  const int64_t round = (int64_t)P * stripe_layout.interleave;
  p.full = cache_len / round;
  p.rem = cache_len % round;
  p.P = P;
  p.interleave = stripe_layout.interleave;
  p.ring_start = stripe_layout.ring_start;
  p.nb = (int32_t)((max_len + ra::kBKV - 1) / ra::kBKV);
  p.nq = NQ;
  p.nkv = NKV;
  p.group = group;
  p.q_rows = C;
  p.real_rows = d.real_rows;
  p.head_rows = d.head_rows;
  p.head_pos = d.head_pos;
  p.tail_pos = d.tail_pos;
  p.row_tiles = (int32_t)((rows_total + ra::kRowsPerWG - 1) / ra::kRowsPerWG);
  p.splits = splits;
  {
    const int64_t t_max = ((regions & RA_REGION_CACHE) ? (int64_t)P * p.nb : 0) +
                          ((regions & RA_REGION_CURRENT) ? max_pos / ra::kBKV + 1 : 0);
    p.seg_tiles = splits == 1 ? (int32_t)(lim31 / 4) : (int32_t)((t_max + splits - 1) / splits);
    if (p.seg_tiles < 1) p.seg_tiles = 1;
  }
  p.seg_out_stride = (int64_t)C * NQ * HD;
  if ((int64_t)p.row_tiles * splits * NKV >= lim31 / 2)
    return fail(RA_ERR_UNSUPPORTED, "too many workgroups");
  p.grid_real = p.row_tiles * splits * NKV;
  p.out_f32 = d.out_dtype == RA_DTYPE_FP32;
  p.store_f32 = p.out_f32 || splits > 1;
  p.regions = regions;
  const float scale = d.scale == 0.f ? 1.f / std::sqrt((float)HD) : d.scale;
  p.scale_log2e = scale * 1.4426950408889634f;
  if ((int64_t)p.nb * P >= lim31)
    return fail(RA_ERR_UNSUPPORTED, "too many ring tiles");
  if (write && write->n_tokens > 0) {
    p.wk_cache = static_cast<uint16_t*>(write->k_cache);
    p.wv_cache = static_cast<uint16_t*>(write->v_cache);
    p.write_pos0 = cache_len;
    p.write_tokens = write->n_tokens;
    p.write_per_wg = (write->n_tokens + p.grid_real - 1) / p.grid_real;
    p.write_chunks = (int32_t)(rowstride / 16);
  }

  log_geometry(p, HD);
  hipError_t e = ra::launch_fused(p, HD, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(RA_ERR_HIP, "fused attention launch failed: %s", hipGetErrorString(e));
  return RA_OK;
}


// ring_attn_prefill_split, with the strided write in the launch when
// `write` is given (its arguments checked by the caller).
int split_impl(const void* q, const void* k_cache, const void* v_cache, const void* k_cur,
               const void* v_cur, int64_t cache_len, int32_t P, ra_stripe_layout_t stripe_layout,
               int32_t splits, void* workspace, int64_t workspace_bytes, void* out, float* lse,
               const ra_dims_t* dims, void* stream, const FusedWrite* write) {
  int64_t need = 0;
  if (int rc = ra_split_workspace_bytes(dims, splits, &need)) return rc;
  if (splits == 1)
    return prefill_regions(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout,
                           RA_REGION_CACHE | RA_REGION_CURRENT, out, lse, dims, stream, 1, write);
  const ra_dims_t& d = *dims;
  if (d.real_rows > 0 && !out) return fail(RA_ERR_INVALID_ARG, "out must not be NULL");
  if (!workspace) return fail(RA_ERR_INVALID_ARG, "workspace must not be NULL when splits > 1");
  if (!aligned16(workspace))
    return fail(RA_ERR_INVALID_ARG, "every tensor pointer must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(RA_ERR_INVALID_ARG, "workspace_bytes %lld is below the %lld bytes splits=%d needs",
                (long long)workspace_bytes, (long long)need, splits);
  // the workspace must not overlap the caller's tensors
  const int64_t C = d.q_rows, NQ = d.num_q_heads, HD = d.head_dim, NKV = d.num_kv_heads;
  struct R { const void* p; int64_t n; };
  // (the caches in full when the launch writes them)
  const int64_t cache_bytes = (cache_len > 0 || write) ? (int64_t)P * d.shard_cap * NKV * HD * 2 : 0;
  const R others[] = {{q, C * NQ * HD * 2}, {k_cache, cache_bytes}, {v_cache, cache_bytes},
                      {k_cur, (int64_t)d.cur_len * NKV * HD * 2}, {v_cur, (int64_t)d.cur_len * NKV * HD * 2},
                      {out, C * NQ * HD * (d.out_dtype == RA_DTYPE_FP32 ? 4 : 2)}, {lse, NQ * C * 4}};
  for (const R& r : others)
    if (overlaps(workspace, need, r.p, r.n))
      return fail(RA_ERR_INVALID_ARG, "workspace overlaps another tensor");
  char* ws = static_cast<char*>(workspace);
  float* part_lse = reinterpret_cast<float*>(ws + split_part_bytes(d, splits));
  if (int rc = prefill_regions(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout,
                               RA_REGION_CACHE | RA_REGION_CURRENT, ws, part_lse, dims, stream,
                               splits, write))
    return rc;
  if (d.real_rows == 0) return RA_OK;
  ra::MergeSplitsParams m{};
  m.part_o = ws;
  m.part_lse = part_lse;
  m.out = out;
  m.lse = lse;
  m.splits = splits;
  m.q_rows = d.q_rows;
  m.real_rows = d.real_rows;
  m.nq = d.num_q_heads;
  m.hd = d.head_dim;
  m.parts_f32 = 1;
  m.out_f32 = d.out_dtype == RA_DTYPE_FP32;
  hipError_t e = ra::launch_merge_splits(m, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(RA_ERR_HIP, "split merge launch failed: %s", hipGetErrorString(e));
  return RA_OK;
}

// The strided write's own checks (those of kv_cache_write, plus what a
// launch that reads and writes the caches at once needs), then the
// attention launch, split or not, carrying the write.
int prefill_write_impl(const void* q, void* k_cache, void* v_cache, const void* k_cur,
                       const void* v_cur, int64_t cache_len, int32_t P,
                       ra_stripe_layout_t stripe_layout, int32_t splits, void* workspace,
                       int64_t workspace_bytes, int32_t n_tokens, void* out, float* lse,
                       const ra_dims_t* dims, void* stream) {
  if (int rc = check_heads(dims)) return rc;
  if (int rc = check_layout(P, stripe_layout, cache_len)) return rc;
  const ra_dims_t& d = *dims;
  if (n_tokens < 0 || n_tokens > d.cur_len)
    return fail(RA_ERR_INVALID_ARG, "n_tokens must be in [0, cur_len=%d]; got %d", d.cur_len,
                n_tokens);
  // no rows to compute: the write alone; nothing to write: the attention alone
  if (d.real_rows == 0)
    return kv_cache_write(k_cur, v_cur, n_tokens, k_cache, v_cache, cache_len, P, stripe_layout,
                          dims, stream);
  if (n_tokens == 0)
    return split_impl(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout, splits,
                      workspace, workspace_bytes, out, lse, dims, stream, nullptr);
  const int64_t end = cache_len + n_tokens;
  const int64_t need = shard_len(end, P, stripe_layout.interleave, 0);
  if (need > d.shard_cap)
    return fail(RA_ERR_INVALID_ARG,
                "writing positions [%lld, %lld) needs %lld slots in shard 0 but shard_cap is %lld",
                (long long)cache_len, (long long)end, (long long)need, (long long)d.shard_cap);
  if (!k_cache || !v_cache)
    return fail(RA_ERR_INVALID_ARG, "k_cache and v_cache must not be NULL when n_tokens > 0");
  // the caches are written: no other tensor may share their bytes
  const int64_t row_bytes = (int64_t)d.num_kv_heads * d.head_dim * 2;
  const int64_t cache_bytes = row_bytes * P * d.shard_cap;
  if (overlaps(k_cache, cache_bytes, v_cache, cache_bytes))
    return fail(RA_ERR_INVALID_ARG, "k_cache and v_cache overlap");
  const int64_t out_bytes = (int64_t)d.q_rows * d.num_q_heads * d.head_dim *
                            (d.out_dtype == RA_DTYPE_FP32 ? 4 : 2);
  struct R { const void* p; int64_t n; };
  const R others[] = {{q, (int64_t)d.q_rows * d.num_q_heads * d.head_dim * 2},
                      {k_cur, row_bytes * d.cur_len}, {v_cur, row_bytes * d.cur_len},
                      {out, out_bytes}, {lse, (int64_t)d.num_q_heads * d.q_rows * 4}};
  for (const R& r : others)
    if (overlaps(k_cache, cache_bytes, r.p, r.n) || overlaps(v_cache, cache_bytes, r.p, r.n))
      return fail(RA_ERR_INVALID_ARG, "a cache tensor overlaps q, k_cur, v_cur, out or lse");
  const FusedWrite w{k_cache, v_cache, n_tokens};
  return split_impl(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout, splits,
                    workspace, workspace_bytes, out, lse, dims, stream, &w);
}

}  // namespace

extern "C" {

int ring_attn_prefill(const void* q, const void* k_cache, const void* v_cache, const void* k_cur,
                      const void* v_cur, int64_t cache_len, int32_t P,
                      ra_stripe_layout_t stripe_layout, void* out, float* lse,
                      const ra_dims_t* dims, void* stream) {
  return prefill_regions(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout,
                         RA_REGION_CACHE | RA_REGION_CURRENT, out, lse, dims, stream);
}

int ring_attn_prefill_write(const void* q, void* k_cache, void* v_cache, const void* k_cur,
                            const void* v_cur, int64_t cache_len, int32_t P,
                            ra_stripe_layout_t stripe_layout, int32_t n_tokens, void* out,
                            float* lse, const ra_dims_t* dims, void* stream) {
  return prefill_write_impl(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout, 1,
                            nullptr, 0, n_tokens, out, lse, dims, stream);
}

int ring_attn_prefill_split_write(const void* q, void* k_cache, void* v_cache, const void* k_cur,
                                  const void* v_cur, int64_t cache_len, int32_t P,
                                  ra_stripe_layout_t stripe_layout, int32_t splits,
                                  void* workspace, int64_t workspace_bytes, int32_t n_tokens,
                                  void* out, float* lse, const ra_dims_t* dims, void* stream) {
  return prefill_write_impl(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout,
                            splits, workspace, workspace_bytes, n_tokens, out, lse, dims, stream);
}

int ring_attn_partial(const void* q, const void* k_cache, const void* v_cache, const void* k_cur,
                      const void* v_cur, int64_t cache_len, int32_t P,
                      ra_stripe_layout_t stripe_layout, int32_t regions, void* out, float* lse,
                      const ra_dims_t* dims, void* stream) {
  if (regions != RA_REGION_CACHE && regions != RA_REGION_CURRENT &&
      regions != (RA_REGION_CACHE | RA_REGION_CURRENT))
    return fail(RA_ERR_INVALID_ARG, "regions must be RA_REGION_CACHE, RA_REGION_CURRENT or both; "
                "got %d", regions);
  return prefill_regions(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout, regions,
                         out, lse, dims, stream);
}

int ra_split_suggest(const ra_dims_t* dims, int32_t num_cus, int32_t* splits) {
  if (int rc = check_heads(dims)) return rc;
  if (num_cus < 1) return fail(RA_ERR_INVALID_ARG, "num_cus must be >= 1; got %d", num_cus);
  if (!splits) return fail(RA_ERR_INVALID_ARG, "splits must not be NULL");
  const ra_dims_t& d = *dims;
  if (d.real_rows < 0 || d.real_rows > d.q_rows)
    return fail(RA_ERR_INVALID_ARG, "real_rows must be in [0, q_rows=%d]; got %d", d.q_rows,
                d.real_rows);
  // One workgroup per CU at a time (two at HD = 64).  A launch of W
  // workgroups takes ceil(W / slots) waves; splitting multiplies W by S at a
  // small cost per segment (its own Q load and partial output), so pick the
  // S that best fills the last wave.
  const int64_t group = d.num_q_heads / d.num_kv_heads;
  const int64_t wgs = ((int64_t)d.real_rows * group + ra::kRowsPerWG - 1) / ra::kRowsPerWG *
                      d.num_kv_heads;
  int32_t best = 1;
  double best_cost = 1e300;
  for (int32_t s = 1; s <= 16 && wgs > 0; ++s) {
    const double waves = (double)(wgs * s) / ((int64_t)num_cus * ra::wgs_per_cu(d.head_dim));
    const double cost = std::ceil(waves) / waves * (1.0 + 0.02 * (s - 1));
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = s;
    }
  }
  *splits = best;
  return RA_OK;
}

int ra_split_workspace_bytes(const ra_dims_t* dims, int32_t splits, int64_t* bytes) {
  if (int rc = check_heads(dims)) return rc;
  if (splits < 1 || splits > RA_MAX_SPLITS)
    return fail(RA_ERR_INVALID_ARG, "splits must be in [1, %d]; got %d", RA_MAX_SPLITS, splits);
  if (dims->q_rows < 0) return fail(RA_ERR_INVALID_ARG, "q_rows must be >= 0");
  if (!bytes) return fail(RA_ERR_INVALID_ARG, "bytes must not be NULL");
  *bytes = splits == 1 ? 0 : split_workspace_bytes(*dims, splits);
  return RA_OK;
}

int ring_attn_prefill_split(const void* q, const void* k_cache, const void* v_cache,
                            const void* k_cur, const void* v_cur, int64_t cache_len, int32_t P,
                            ra_stripe_layout_t stripe_layout, int32_t splits, void* workspace,
                            int64_t workspace_bytes, void* out, float* lse,
                            const ra_dims_t* dims, void* stream) {
  return split_impl(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout, splits,
                    workspace, workspace_bytes, out, lse, dims, stream, nullptr);
}

}  // extern "C"

namespace {

// Workspace of ring_attn_prefill_split_noalloc: one array per GPU in the
// library's own device memory, reserved when the code object is loaded and
// held until the process ends.  Host code must not use this name as an
// address (on the host it stands in for the symbol only); it uses the
// device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[RA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device

// The current device's copy of `scratch`, looked up once per device.
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RA_ERR_UNSUPPORTED, "device %d is past the %d devices this build supports", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(RA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RA_OK;
}

}  // namespace

extern "C" {

int ring_attn_prefill_split_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const void* k_cur, const void* v_cur, int64_t cache_len,
                                    int32_t P, ra_stripe_layout_t stripe_layout, int32_t splits,
                                    void* out, float* lse, const ra_dims_t* dims, void* stream) {
  int64_t need = 0;
  if (int rc = ra_split_workspace_bytes(dims, splits, &need)) return rc;
  if (need > RA_NOALLOC_SCRATCH_BYTES)
    return fail(RA_ERR_UNSUPPORTED,
                "splits=%d over q_rows=%d x num_q_heads=%d x head_dim=%d needs %lld bytes of "
                "workspace; the library's own holds %lld (use ring_attn_prefill_split with a "
                "workspace of your own)",
                splits, dims->q_rows, dims->num_q_heads, dims->head_dim, (long long)need,
                (long long)RA_NOALLOC_SCRATCH_BYTES);
  if (splits == 1)
    return ring_attn_prefill(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout,
                             out, lse, dims, stream);
  void* ws = nullptr;
  if (int rc = scratch_on_current_device(&ws)) return rc;
  return ring_attn_prefill_split(q, k_cache, v_cache, k_cur, v_cur, cache_len, P, stripe_layout,
                                 splits, ws, RA_NOALLOC_SCRATCH_BYTES, out, lse, dims, stream);
}

int merge_attn_states(const void* o1, const float* lse1, const void* o2, const float* lse2,
                      int32_t parts_dtype, void* out, float* lse, const ra_dims_t* dims,
                      void* stream) {
  if (!dims) return fail(RA_ERR_INVALID_ARG, "dims must not be NULL");
  const ra_dims_t& d = *dims;
  if (d.num_q_heads < 1) return fail(RA_ERR_INVALID_ARG, "num_q_heads must be >= 1; got %d",
                                     d.num_q_heads);
  if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256)
    return fail(RA_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256; got %d", d.head_dim);
  if (d.q_rows < 0) return fail(RA_ERR_INVALID_ARG, "q_rows must be >= 0; got %d", d.q_rows);
  if (d.real_rows < 0 || d.real_rows > d.q_rows)
    return fail(RA_ERR_INVALID_ARG, "real_rows must be in [0, q_rows=%d]; got %d", d.q_rows,
                d.real_rows);
  if (d.out_dtype != RA_DTYPE_BF16 && d.out_dtype != RA_DTYPE_FP32)
    return fail(RA_ERR_INVALID_ARG, "out_dtype must be RA_DTYPE_BF16 or RA_DTYPE_FP32; got %d",
                d.out_dtype);
  if (parts_dtype != RA_DTYPE_BF16 && parts_dtype != RA_DTYPE_FP32)
    return fail(RA_ERR_INVALID_ARG, "parts_dtype must be RA_DTYPE_BF16 or RA_DTYPE_FP32; got %d",
                parts_dtype);
  if ((int64_t)d.q_rows * d.num_q_heads * d.head_dim >= ((int64_t)1 << 40))
    return fail(RA_ERR_UNSUPPORTED, "q_rows * num_q_heads * head_dim is too large");
  if (d.real_rows == 0) return RA_OK;
  if (!o1 || !lse1 || !o2 || !lse2 || !out)
    return fail(RA_ERR_INVALID_ARG, "o1, lse1, o2, lse2 and out must not be NULL");
  const void* ptrs[] = {o1, lse1, o2, lse2, out, lse};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr))
      return fail(RA_ERR_INVALID_ARG, "every tensor pointer must be 16-byte aligned");
  const int64_t elems = (int64_t)d.q_rows * d.num_q_heads * d.head_dim;
  const int64_t o_bytes = elems * (parts_dtype == RA_DTYPE_FP32 ? 4 : 2);
  const int64_t l_bytes = (int64_t)d.q_rows * d.num_q_heads * 4;
  const int64_t out_bytes = elems * (d.out_dtype == RA_DTYPE_FP32 ? 4 : 2);
  struct R { const void* p; int64_t n; };
  const R ins[] = {{o1, o_bytes}, {lse1, l_bytes}, {o2, o_bytes}, {lse2, l_bytes}};
  for (const R& r : ins) {
    if (overlaps(out, out_bytes, r.p, r.n))
      return fail(RA_ERR_INVALID_ARG, "out overlaps an input tensor");
    if (overlaps(lse, l_bytes, r.p, r.n))
      return fail(RA_ERR_INVALID_ARG, "lse overlaps an input tensor");
  }
  if (overlaps(out, out_bytes, lse, l_bytes))
    return fail(RA_ERR_INVALID_ARG, "out and lse overlap");
  ra::MergeParams p{};
  p.o1 = o1;
  p.lse1 = lse1;
  p.o2 = o2;
  p.lse2 = lse2;
  p.out = out;
  p.lse = lse;
  p.q_rows = d.q_rows;
  p.real_rows = d.real_rows;
  p.nq = d.num_q_heads;
  p.hd = d.head_dim;
  p.parts_f32 = parts_dtype == RA_DTYPE_FP32;
  p.out_f32 = d.out_dtype == RA_DTYPE_FP32;
  hipError_t e = ra::launch_merge(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(RA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return RA_OK;
}

int kv_cache_write(const void* k_cur, const void* v_cur, int32_t n_tokens, void* k_cache,
                   void* v_cache, int64_t cache_len, int32_t P, ra_stripe_layout_t stripe_layout,
                   const ra_dims_t* dims, void* stream) {
  if (int rc = check_heads(dims)) return rc;
  if (int rc = check_layout(P, stripe_layout, cache_len)) return rc;
  if (n_tokens < 0) return fail(RA_ERR_INVALID_ARG, "n_tokens must be >= 0; got %d", n_tokens);
  const ra_dims_t& d = *dims;
  const int64_t end = cache_len + n_tokens;
  const int64_t need = shard_len(end, P, stripe_layout.interleave, 0);
  if (need > d.shard_cap)
    return fail(RA_ERR_INVALID_ARG,
                "writing positions [%lld, %lld) needs %lld slots in shard 0 but shard_cap is %lld",
                (long long)cache_len, (long long)end, (long long)need, (long long)d.shard_cap);
  if (n_tokens == 0) return RA_OK;
  if (!k_cur || !v_cur || !k_cache || !v_cache)
    return fail(RA_ERR_INVALID_ARG, "k_cur, v_cur, k_cache and v_cache must not be NULL");
  const void* ptrs[] = {k_cur, v_cur, k_cache, v_cache};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr))
      return fail(RA_ERR_INVALID_ARG, "every tensor pointer must be 16-byte aligned");
  const int64_t row_bytes = (int64_t)d.num_kv_heads * d.head_dim * 2;
  const int64_t cur_bytes = row_bytes * n_tokens;
  const int64_t cache_bytes = row_bytes * P * d.shard_cap;
  if (overlaps(k_cache, cache_bytes, v_cache, cache_bytes))
    return fail(RA_ERR_INVALID_ARG, "k_cache and v_cache overlap");
  const void* curs[] = {k_cur, v_cur};
  for (const void* c : curs)
    if (overlaps(k_cache, cache_bytes, c, cur_bytes) || overlaps(v_cache, cache_bytes, c, cur_bytes))
      return fail(RA_ERR_INVALID_ARG, "a cache tensor overlaps k_cur or v_cur");

  ra::WriteParams p{};
  p.k_cur = static_cast<const uint16_t*>(k_cur);
  p.v_cur = static_cast<const uint16_t*>(v_cur);
  p.k_cache = static_cast<uint16_t*>(k_cache);
  p.v_cache = static_cast<uint16_t*>(v_cache);
  p.cache_len = cache_len;
  p.shard_cap = d.shard_cap;
  p.n_tokens = n_tokens;
  p.P = P;
  p.interleave = stripe_layout.interleave;
  p.row_chunks = (int32_t)(row_bytes / 16);
  hipError_t e = ra::launch_kv_cache_write(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(RA_ERR_HIP, "kv_cache_write launch failed: %s", hipGetErrorString(e));
  return RA_OK;
}

}  // extern "C"
