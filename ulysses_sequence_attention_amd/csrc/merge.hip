// Merge of partial attention results over key blocks by their log-sum-exp
// (flashdreams cp.py, ContextParallelAttention, ring path: the running result
// takes in each block's output with a logistic weight of the LSE difference,
// and its LSE becomes the log of the summed exponentials).  Taking in n
// blocks one after the other is, in exact arithmetic, one weighted sum:
//   L = log sum_i exp(lse_i),  out = sum_i exp(lse_i - L) out_i,
// which this kernel evaluates in fp32 in one pass (max-shifted, so no
// overflow; a block with lse = -inf has weight 0).
//
// HBM stream: one thread per one or two 16-byte chunks (8 bf16 each) of the
// output; it reads the same chunks of every part and the n LSEs of its
// (b, h, row), which the threads of that row share through the cache.
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
// (b, row, head) when known at compile time (0 = runtime head_dim / 8); U:
// consecutive chunks per thread (1 or 2; 2 when CPR is even), which shares a
// row's LSE loads and weights between them and doubles the loads in flight.
template <typename IDX, int CPR, int U>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(MergeArgs a) {
  const IDX cpr = CPR ? (IDX)CPR : (IDX)(a.head_dim / 8);
  const IDX units = cpr / U;
  const IDX total = (IDX)a.batch * (IDX)a.rows * (IDX)a.heads * units;
  const IDX idx = (IDX)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const IDX cu = idx % units;
  const IDX r2 = idx / units;
  const IDX h = r2 % (IDX)a.heads;
  const IDX br = r2 / (IDX)a.heads;
  const IDX row = br % (IDX)a.rows;
  const IDX b = br / (IDX)a.rows;
  const size_t li = ((size_t)b * a.heads + h) * a.rows + row;
  const IDX c0 = r2 * cpr + cu * U;   // first 16-byte chunk of this thread

  // All loads first (the LSEs and the output chunks are independent), so one
  // memory round trip covers the thread's whole input.  Plain loads: partial
  // results are usually still in the caches (nontemporal loads measured
  // slower).
  float lv[kMaxMergeParts];
  u32x4 xs[kMaxMergeParts][U];
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i) {
    if (i < a.n) {
      lv[i] = a.lse[i][li];
#pragma unroll
      for (int u = 0; u < U; ++u) xs[i][u] = ((const u32x4*)a.o[i])[c0 + u];
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxMergeParts; ++i)
    if (i < a.n) m = fmaxf(m, lv[i]);
  float acc[U][8];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[u][j] = 0.0f;
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
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const u32x4 x = xs[i][u];
          acc[u][0] += w * bf16_lo(x.x); acc[u][1] += w * bf16_hi(x.x);
          acc[u][2] += w * bf16_lo(x.y); acc[u][3] += w * bf16_hi(x.y);
          acc[u][4] += w * bf16_lo(x.z); acc[u][5] += w * bf16_hi(x.z);
          acc[u][6] += w * bf16_lo(x.w); acc[u][7] += w * bf16_hi(x.w);
        }
      }
    }
    L = m + logf(s);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    u32x4 y;
    y.x = bf16_pair(acc[u][0], acc[u][1]);
    y.y = bf16_pair(acc[u][2], acc[u][3]);
    y.z = bf16_pair(acc[u][4], acc[u][5]);
    y.w = bf16_pair(acc[u][6], acc[u][7]);
    ((u32x4*)a.out)[c0 + u] = y;
  }
  if (a.lse_out != nullptr && cu == 0) a.lse_out[li] = L;
}

}  // namespace

hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s) {
  const long chunks = (long)a.batch * a.rows * a.heads * (a.head_dim / 8);
  auto grid = [&](long threads) { return dim3((unsigned)((threads + kThreads - 1) / kThreads)); };
  if (chunks >= (1L << 32) - kThreads)
    hipLaunchKernelGGL((lse_merge_kernel<size_t, 0, 1>), grid(chunks), dim3(kThreads), 0, s, a);
  else if (a.head_dim == 128)
    hipLaunchKernelGGL((lse_merge_kernel<unsigned, 16, 2>), grid(chunks / 2), dim3(kThreads), 0, s, a);
  else if (a.head_dim == 64)
    hipLaunchKernelGGL((lse_merge_kernel<unsigned, 8, 2>), grid(chunks / 2), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((lse_merge_kernel<unsigned, 0, 1>), grid(chunks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ulys
