// Merge of partial attention results over key blocks by their log-sum-exp
// (flashdreams cp.py, ContextParallelAttention._impl_ring: each step's
// (out, lse) is absorbed with weights sigmoid(lse - prev_lse), and the LSE
// grows by -logsigmoid(prev_lse - lse)).  Absorbing n blocks one after the
// other is, in exact arithmetic, one weighted sum:
//   L = log sum_i exp(lse_i),  out = sum_i exp(lse_i - L) out_i,
// which this kernel evaluates in fp32 in one pass (max-shifted, so no
// overflow; a block with lse = -inf has weight 0).
//
// HBM stream: one thread per 16-byte chunk (8 bf16) of the output; it reads
// the same chunk of every part and the n LSEs of its (b, h, row), which the
// D/8 threads of that row share through the cache.
#include "internal.h"

namespace ulys {
namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

// two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ unsigned int bf16_pair(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, bf16x2));
}

// IDX: index type (32-bit when the chunk count fits); CPR: 16-byte chunks per
// (b, row, head) when known at compile time (0 = runtime head_dim / 8).
template <typename IDX, int CPR>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(MergeArgs a) {
  const IDX cpr = CPR ? (IDX)CPR : (IDX)(a.head_dim / 8);
  const IDX total = (IDX)a.batch * (IDX)a.rows * (IDX)a.heads * cpr;
  const IDX idx = (IDX)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const IDX c = idx % cpr;
  const IDX r2 = idx / cpr;
  const IDX h = r2 % (IDX)a.heads;
  const IDX br = r2 / (IDX)a.heads;
  const IDX row = br % (IDX)a.rows;
  const IDX b = br / (IDX)a.rows;
  const size_t li = ((size_t)b * a.heads + h) * a.rows + row;

  // All loads first (the LSEs and the output chunks are independent), so one
  // memory round trip covers the thread's whole input.
  float lv[kMaxMergeParts];
  u32x4 xs[kMaxMergeParts];
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i) {
    if (i < a.n) {
      lv[i] = a.lse[i][li];
      xs[i] = ((const u32x4*)a.o[i])[idx];
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i)
    if (i < a.n) m = fmaxf(m, lv[i]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  if (m != -INFINITY) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxMergeParts; ++i) {
      if (i < a.n) {
        lv[i] = expf(lv[i] - m);
        s += lv[i];
      }
    }
    const float inv = 1.0f / s;
#pragma unroll
    for (int i = 0; i < kMaxMergeParts; ++i) {
      if (i < a.n) {
        const float w = lv[i] * inv;
        const u32x4 x = xs[i];
        acc[0] += w * bf16_lo(x.x); acc[1] += w * bf16_hi(x.x);
        acc[2] += w * bf16_lo(x.y); acc[3] += w * bf16_hi(x.y);
        acc[4] += w * bf16_lo(x.z); acc[5] += w * bf16_hi(x.z);
        acc[6] += w * bf16_lo(x.w); acc[7] += w * bf16_hi(x.w);
      }
    }
    L = m + logf(s);
  }
  u32x4 y;
  y.x = bf16_pair(acc[0], acc[1]);
  y.y = bf16_pair(acc[2], acc[3]);
  y.z = bf16_pair(acc[4], acc[5]);
  y.w = bf16_pair(acc[6], acc[7]);
  ((u32x4*)a.out)[idx] = y;
  if (a.lse_out != nullptr && c == 0) a.lse_out[li] = L;
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s) {
  const long total = (long)a.batch * a.rows * a.heads * (a.head_dim / 8);
  const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
  if (total >= (1L << 32) - kThreads)
    hipLaunchKernelGGL((lse_merge_kernel<size_t, 0>), grid, dim3(kThreads), 0, s, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL((lse_merge_kernel<unsigned, 16>), grid, dim3(kThreads), 0, s, a);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL((lse_merge_kernel<unsigned, 8>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((lse_merge_kernel<unsigned, 0>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ulys
