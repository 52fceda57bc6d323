// Layout repack kernels: pack (shards -> head-group receive slots, optional
// e4m3fn q/k), unpack (output slot -> shards) and amax (per-tensor fp8 scale
// source).  All three are HBM streams: every thread moves whole 16-byte
// chunks, consecutive lanes take consecutive chunks of one contiguous run
// (a row's Gh*D elements), so each wave reads and writes whole cache lines.
//
// Row map (sglang PR #43521 "Receive slots"/"Layouts"; flashdreams cp.py
// _impl_ulysses): joint row t of rank r comes from
//   prefix: t <  R      -> shard r, row t                 (its own replicated copy)
//           t >= R      -> shard (t-R)/S_l, row R + (t-R)%S_l
//   suffix: t <  P*S_l  -> shard t/S_l, row t%S_l
//           t >= P*S_l  -> shard r, row S_l + (t - P*S_l)
// A K/V-only prefix (sglang layer.py _forward_with_replicated_kv_prefix) is
// the prefix map for k/v and the map without replicated rows for q and o.
#include "internal.h"

namespace ulys {
namespace {

constexpr int kThreads = 256;
// Access forms and chunks per thread, chosen by measurement on MI355X (Wan
// Ulysses-4 shapes): pack reads nontemporal and writes plainly, two chunks
// per thread; unpack reads and writes nontemporal, two chunks per thread.
#ifndef ULYS_PK_NTLOAD
#define ULYS_PK_NTLOAD 1
#endif
#ifndef ULYS_PK_NTSTORE
#define ULYS_PK_NTSTORE 0
#endif
#ifndef ULYS_UP_NTLOAD
#define ULYS_UP_NTLOAD 1
#endif
#ifndef ULYS_UP_NTSTORE
#define ULYS_UP_NTSTORE 1
#endif
#ifndef ULYS_PK_UNROLL
#define ULYS_PK_UNROLL 2
#endif
#ifndef ULYS_UP_UNROLL
#define ULYS_UP_UNROLL 2
#endif
constexpr int kPackUnroll = ULYS_PK_UNROLL;     // chunks per pack thread
constexpr int kUnpackUnroll = ULYS_UP_UNROLL;   // chunks per unpack thread

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void src_of_row(const RepackGeom& g, int rank_of_rep, int t, int* p, int* row) {
  const int body = g.degree * g.s_local;
  if (g.rep_first) {
    if (t < g.n_rep) { *p = rank_of_rep; *row = t; }
    else { const int u = t - g.n_rep; *p = u / g.s_local; *row = g.n_rep + u % g.s_local; }
  } else {
    if (t < body) { *p = t / g.s_local; *row = t % g.s_local; }
    else { *p = rank_of_rep; *row = g.s_local + (t - body); }
  }
}

__device__ __forceinline__ float bf16_to_f32(unsigned int bits16) {
  return __uint_as_float(bits16 << 16);
}

// e4m3fn codes of 4 floats (already scaled), saturated to +-448, round to nearest even.
__device__ __forceinline__ unsigned int pack4_e4m3(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.0f), 448.0f);
  b = fminf(fmaxf(b, -448.0f), 448.0f);
  c = fminf(fmaxf(c, -448.0f), 448.0f);
  d = fminf(fmaxf(d, -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);   // bytes 0,1
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);         // bytes 2,3
  return (unsigned int)w;
}

__device__ __forceinline__ unsigned int e4m3_of_bf16x4(unsigned int lo, unsigned int hi, float inv) {
  return pack4_e4m3(bf16_to_f32(lo & 0xffffu) * inv, bf16_to_f32(lo >> 16) * inv,
                    bf16_to_f32(hi & 0xffffu) * inv, bf16_to_f32(hi >> 16) * inv);
}

// Streaming accesses: every byte is touched once; the nontemporal forms keep
// it from displacing cache lines other work could reuse.
template <bool NT>
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load((const u32x4*)p);
  else return *(const u32x4*)p;
}
template <bool NT>
__device__ __forceinline__ void st_stream(void* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, (u32x4*)p);
  else *(u32x4*)p = v;
}

// grid.x: 16-byte output chunks of one slot [B * rows * cpr], kPackUnroll * kThreads
// per block, thread i taking chunks i, i + kThreads, ...; grid.y = tensor * ngroups
// + group.  All loads of a thread are issued before its stores.  Chunk indices
// are 32-bit (the host rejects slots of 2^32 chunks or more).
__global__ __launch_bounds__(kThreads) void pack_kernel(PackArgs a) {
  const int tensor = blockIdx.y / a.g[0].ngroups;
  const RepackGeom& g = a.g[tensor];
  const int gi = blockIdx.y % g.ngroups;
  const int gh = a.gh[tensor];
  const int D = g.head_dim;
  const int fp8 = a.fp8[tensor];
  const int elems_per_chunk = fp8 ? 16 : 8;       // output chunk is always 16 bytes
  const unsigned cpr = (unsigned)(gh * D / elems_per_chunk);   // chunks per slot row
  const unsigned total = (unsigned)g.batch * (unsigned)g.rows * cpr;
  const int H = a.heads[tensor];
  const int hbase = a.h0[tensor] + gi * gh;
  float inv = 1.0f;
  if (fp8) {
    const float am = a.amax[tensor];
    inv = am > 0.0f ? __fdiv_rn(448.0f, am) : 1.0f;
  }
  unsigned char* dst_base = (unsigned char*)a.dst[tensor] +
                            (size_t)gi * g.batch * g.rows * gh * D * (fp8 ? 1 : 2);
  const unsigned first = blockIdx.x * (kPackUnroll * kThreads) + threadIdx.x;
  u32x4 x0[kPackUnroll], x1[kPackUnroll];
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    const unsigned idx = first + u * kThreads;
    if (idx < total) {
      const unsigned c = idx % cpr;
      const unsigned bt = idx / cpr;
      const unsigned t = bt % (unsigned)g.rows;
      const unsigned b = bt / (unsigned)g.rows;
      int p, srow;
      src_of_row(g, g.rank, (int)t, &p, &srow);
      const uint16_t* src = a.src[tensor][p] +
                            (((size_t)b * g.shard_rows + srow) * H + hbase) * D + (size_t)c * elems_per_chunk;
      x0[u] = ld_stream<ULYS_PK_NTLOAD>(src);
      if (fp8) x1[u] = ld_stream<ULYS_PK_NTLOAD>(src + 8);
    }
  }
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    const unsigned idx = first + u * kThreads;
    if (idx < total) {
      u32x4 y = x0[u];
      if (fp8) {
        y.x = e4m3_of_bf16x4(x0[u].x, x0[u].y, inv);
        y.y = e4m3_of_bf16x4(x0[u].z, x0[u].w, inv);
        y.z = e4m3_of_bf16x4(x1[u].x, x1[u].y, inv);
        y.w = e4m3_of_bf16x4(x1[u].z, x1[u].w, inv);
      }
      st_stream<ULYS_PK_NTSTORE>(dst_base + (size_t)idx * 16, y);
    }
  }
}

// grid.x: chunks of [B * shard_rows * cpr] (as pack); grid.y = p * ngroups + group
__global__ __launch_bounds__(kThreads) void unpack_kernel(UnpackArgs a) {
  const RepackGeom& g = a.g;
  const int p = blockIdx.y / g.ngroups;
  const int gi = blockIdx.y % g.ngroups;
  const int D = g.head_dim;
  const unsigned cpr = (unsigned)(a.gh * D / 8);
  const unsigned total = (unsigned)g.batch * (unsigned)g.shard_rows * cpr;
  const int hbase = a.h0 + gi * a.gh;
  const uint16_t* src_base = a.src + (size_t)gi * g.batch * g.rows * a.gh * D;
  const unsigned first = blockIdx.x * (kUnpackUnroll * kThreads) + threadIdx.x;
  u32x4 x[kUnpackUnroll];
  uint16_t* dst[kUnpackUnroll];
#pragma unroll
  for (int u = 0; u < kUnpackUnroll; ++u) {
    const unsigned idx = first + u * kThreads;
    dst[u] = nullptr;
    if (idx < total) {
      const unsigned c = idx % cpr;
      const unsigned br = idx / cpr;
      const int r = (int)(br % (unsigned)g.shard_rows);      // row within shard p
      const unsigned b = br / (unsigned)g.shard_rows;
      int t;
      if (g.rep_first) t = (r < g.n_rep) ? r : g.n_rep + p * g.s_local + (r - g.n_rep);
      else t = (r < g.s_local) ? p * g.s_local + r : g.degree * g.s_local + (r - g.s_local);
      x[u] = ld_stream<ULYS_UP_NTLOAD>(src_base + (((size_t)b * g.rows + t) * a.gh) * D + (size_t)c * 8);
      dst[u] = a.dst[p] + (((size_t)b * g.shard_rows + r) * a.heads + hbase) * D + (size_t)c * 8;
    }
  }
#pragma unroll
  for (int u = 0; u < kUnpackUnroll; ++u)
    if (first + u * kThreads < total) st_stream<ULYS_UP_NTSTORE>(dst[u], x[u]);
}

__global__ void amax_zero_kernel(unsigned int* out) {
  if (threadIdx.x == 0) *out = 0u;
}

__global__ __launch_bounds__(kThreads) void amax_kernel(AmaxArgs a) {
  unsigned int m = 0;
  const size_t total = (size_t)a.n * a.chunks_each;
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += stride) {
    const int tsr = (int)(idx / a.chunks_each);
    const size_t c = idx % a.chunks_each;
    const u32x4 x = ((const u32x4*)a.src[tsr])[c];
    // |bf16| ordered as its 15 magnitude bits (finite inputs)
    m = max(m, max(max(x.x & 0x7fffu, (x.x >> 16) & 0x7fffu), max(x.y & 0x7fffu, (x.y >> 16) & 0x7fffu)));
    m = max(m, max(max(x.z & 0x7fffu, (x.z >> 16) & 0x7fffu), max(x.w & 0x7fffu, (x.w >> 16) & 0x7fffu)));
  }
  for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned int)__shfl_xor((int)m, off, 64));
  __shared__ unsigned int red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned int r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = max(r, red[i]);
    atomicMax(a.out, r << 16);   // non-negative float bits order like unsigned ints
  }
}

}  // namespace

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  // the largest chunk count over the three tensors sets grid.x
  long most = 0;
  for (int t = 0; t < 3; ++t) {
    const long cpr = (long)a.gh[t] * a.g[t].head_dim / (a.fp8[t] ? 16 : 8);
    const long total = (long)a.g[t].batch * a.g[t].rows * cpr;
    if (total > most) most = total;
  }
  const long per_block = (long)kThreads * kPackUnroll;
  dim3 grid((unsigned)((most + per_block - 1) / per_block), 3 * a.g[0].ngroups);
  hipLaunchKernelGGL(pack_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_unpack(const UnpackArgs& a, hipStream_t s) {
  const long total = (long)a.g.batch * a.g.shard_rows * (a.gh * a.g.head_dim / 8);
  const long per_block = (long)kThreads * kUnpackUnroll;
  dim3 grid((unsigned)((total + per_block - 1) / per_block), a.g.degree * a.g.ngroups);
  hipLaunchKernelGGL(unpack_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_amax(const AmaxArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(amax_zero_kernel, dim3(1), dim3(64), 0, s, a.out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t total = (size_t)a.n * a.chunks_each;
  size_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 2048) blocks = 2048;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ulys
