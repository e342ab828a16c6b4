// Strided KV-cache write for gfx950.
//
// Method: vLLM tpu-inference pull request "PCP: in-kernel ring cache phase,
// fused with the current phase", Design section (each rank's cache is a
// striped shard) and Testing section (the strided KV-cache write is
// bit-exact).  Current token t at global position p = cache_len + t goes to
// shard (p / I) mod P, slot ((p / I) / P) * I + p mod I, copied bit for bit.
//
// One thread moves one 16-byte chunk of a token row for both K and V, so a
// wavefront reads 1 KiB of contiguous source and writes whole 16-byte-aligned
// runs of each destination row: every access is a full 128-bit transaction.
// The position map is evaluated once per chunk with 64-bit integer math.
#include "ra_internal.h"

namespace ra {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void kv_cache_write_kernel(WriteParams p) {
  const int64_t total = (int64_t)p.n_tokens * p.row_chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t t = idx / p.row_chunks;
    const int c = (int)(idx - t * p.row_chunks);
    const int64_t pos = p.cache_len + t;
    const int64_t unit = pos / p.interleave;
    const int64_t shard = unit % p.P;
    const int64_t slot = (unit / p.P) * p.interleave + (pos - unit * p.interleave);
    const int64_t dst = (shard * p.shard_cap + slot) * p.row_chunks + c;
    const int64_t src = t * p.row_chunks + c;
    const i32x4 kx = reinterpret_cast<const i32x4*>(p.k_cur)[src];
    const i32x4 vx = reinterpret_cast<const i32x4*>(p.v_cur)[src];
    reinterpret_cast<i32x4*>(p.k_cache)[dst] = kx;
    reinterpret_cast<i32x4*>(p.v_cache)[dst] = vx;
  }
}

}  // namespace

hipError_t launch_kv_cache_write(const WriteParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.n_tokens * p.row_chunks;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ra
