// Log-sum-exp merge of two partial attentions over disjoint key sets, for
// gfx950.
//
// Method: vLLM tpu-inference pull request "PCP: in-kernel ring cache phase,
// fused with the current phase", Summary section: the removed two-launch
// variant ran a cache-only ring launch and the current phase separately and
// combined them with an LSE merge (merge_attn_states).  Kept here as the
// comparator of the fused launch.  For each real row and query head:
//     lse = log(exp(lse1) + exp(lse2)),
//     out = exp(lse1 - lse) * o1 + exp(lse2 - lse) * o2,
// with a part whose lse is -inf (it saw no key) weighted 0, and out = 0,
// lse = -inf when both are.
//
// HBM bound: per (row, head) it reads 2 x HD partial outputs (bf16 or fp32)
// and writes HD outputs.  A thread moves four consecutive elements;
// consecutive threads cover consecutive elements, so every wavefront access
// is contiguous.
#include "ra_internal.h"

namespace ra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void merge_attn_states_kernel(MergeParams p) {
  const int quads = p.hd / 4;                          // 16-byte groups per (row, head)
  const int64_t total = (int64_t)p.real_rows * p.nq * quads;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t rh = idx / quads;                    // row * NQ + head
    const int row = (int)(rh / p.nq), h = (int)(rh - (int64_t)row * p.nq);
    const int64_t li = (int64_t)h * p.q_rows + row;
    const float l1 = p.lse1[li], l2 = p.lse2[li];
    const float m = fmaxf(l1, l2);
    float w1 = 0.f, w2 = 0.f, lse = m;                 // m = -inf: neither part saw a key
    if (m != -__builtin_inff()) {
      const float e1 = __expf(l1 - m), e2 = __expf(l2 - m);  // exp(-inf) = 0
      const float s = e1 + e2;
      w1 = e1 / s;
      w2 = e2 / s;
      lse = m + __logf(s);
    }
    const int64_t e = idx * 4;                         // element offset of this group
    f32x4 a, b;
    if (p.parts_f32) {
      a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.o1) + e);
      b = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.o2) + e);
    } else {
      const bf16x4 x = *reinterpret_cast<const bf16x4*>(static_cast<const uint16_t*>(p.o1) + e);
      const bf16x4 y = *reinterpret_cast<const bf16x4*>(static_cast<const uint16_t*>(p.o2) + e);
      a = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
      b = f32x4{(float)y[0], (float)y[1], (float)y[2], (float)y[3]};
    }
    const f32x4 o = {w1 * a[0] + w2 * b[0], w1 * a[1] + w2 * b[1], w1 * a[2] + w2 * b[2],
                     w1 * a[3] + w2 * b[3]};
    if (p.out_f32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + e) = o;
    } else {
      const bf16x4 ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
      *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.out) + e) = ob;
    }
    if (p.lse != nullptr && idx % quads == 0) p.lse[li] = lse;
  }
}

// The same merge over the S partials of a split launch (segments of one
// row's key walk): lse = log sum_s exp(lse_s), out = sum_s exp(lse_s - lse) o_s.
__global__ __launch_bounds__(256) void merge_splits_kernel(MergeSplitsParams p) {
  const int quads = p.hd / 4;
  const int64_t total = (int64_t)p.real_rows * p.nq * quads;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t part_stride = (int64_t)p.q_rows * p.nq * p.hd;      // elements per partial
  const int64_t lse_stride = (int64_t)p.nq * p.q_rows;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int64_t rh = idx / quads;
    const int row = (int)(rh / p.nq), h = (int)(rh - (int64_t)row * p.nq);
    const int64_t li = (int64_t)h * p.q_rows + row;
    float m = -__builtin_inff();
    for (int s = 0; s < p.splits; ++s) m = fmaxf(m, p.part_lse[s * lse_stride + li]);
    const int64_t e = idx * 4;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    float lse = m;
    if (m != -__builtin_inff()) {
      float sum = 0.f;
      for (int s = 0; s < p.splits; ++s) {
        const float w = __expf(p.part_lse[s * lse_stride + li] - m);  // exp(-inf) = 0
        sum += w;
        f32x4 a;
        if (p.parts_f32) {
          a = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.part_o) +
                                              s * part_stride + e);
        } else {
          const bf16x4 x = *reinterpret_cast<const bf16x4*>(
              static_cast<const uint16_t*>(p.part_o) + s * part_stride + e);
          a = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
        }
        o = f32x4{o[0] + w * a[0], o[1] + w * a[1], o[2] + w * a[2], o[3] + w * a[3]};
      }
      const float inv = 1.f / sum;
      o = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
      lse = m + __logf(sum);
    }
    if (p.out_f32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + e) = o;
    } else {
      const bf16x4 ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
      *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(p.out) + e) = ob;
    }
    if (p.lse != nullptr && idx % quads == 0) p.lse[li] = lse;
  }
}

}  // namespace

hipError_t launch_merge_splits(const MergeSplitsParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.real_rows * p.nq * (p.hd / 4);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  hipLaunchKernelGGL(merge_splits_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.real_rows * p.nq * (p.hd / 4);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 16384 ? blocks : 16384);
  hipLaunchKernelGGL(merge_attn_states_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ra
