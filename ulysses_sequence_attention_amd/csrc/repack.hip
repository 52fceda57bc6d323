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
// Chunks (16 bytes) per thread, chunk order and access forms, chosen by
// sweeping them on MI355X at the Wan Ulysses-4 rank shapes with two rotating
// slot sets (nothing cache-resident):
//  * pack, bf16 tensors: two chunks per thread, the chunks of one slot in
//    order (contiguous writes), nontemporal loads and stores;
//  * pack, e4m3 tensors: two chunks per thread, a joint row's chunks group
//    after group (contiguous reads), nontemporal loads, plain stores;
//  * unpack: one chunk per thread, a shard row's chunks group after group
//    (contiguous writes), nontemporal loads, plain stores (+10% over
//    nontemporal stores);
//  * amax: eight chunks per thread in flight, 1024 workgroups in all.
constexpr int kPackUnroll = 2;
constexpr int kUnpackUnroll = 1;
constexpr int kAmaxUnroll = 8;
constexpr int kAmaxBlocks = 1024;

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

// grid.x: 16-byte output chunks of one tensor's slots [ngroups][B * rows * cpr], kPackUnroll * kThreads
// per block, thread i taking chunks i, i + kThreads, ...; grid.y = tensor.  bf16 tensors take the chunks
// slot after slot (consecutive lanes write one contiguous run of a slot); e4m3 tensors take a joint row's
// chunks group after group (consecutive lanes read one contiguous run of the source row, the launch's
// heads).  All loads of a thread are issued before its stores.  Chunk indices are 32-bit (the host
// rejects slots of 2^32 chunks or more).
__global__ __launch_bounds__(kThreads) void pack_kernel(PackArgs a) {
  const int tensor = blockIdx.y;
  const RepackGeom& g = a.g[tensor];
  const int gh = a.gh[tensor];
  const int D = g.head_dim;
  const int fp8 = a.fp8[tensor];
  const int elems_per_chunk = fp8 ? 16 : 8;       // output chunk is always 16 bytes
  const unsigned cpr = (unsigned)(gh * D / elems_per_chunk);   // chunks per slot row of one group
  const unsigned cpr_all = cpr * (unsigned)g.ngroups;          // chunks per joint row, all groups
  const unsigned per_slot = (unsigned)g.batch * (unsigned)g.rows * cpr;
  const unsigned total = per_slot * (unsigned)g.ngroups;
  const int H = a.heads[tensor];
  const int hbase = a.h0[tensor];
  float inv = 1.0f;
  if (fp8) {
    const float am = a.amax[tensor];
    inv = am > 0.0f ? __fdiv_rn(448.0f, am) : 1.0f;
  }
  const unsigned first = blockIdx.x * (kPackUnroll * kThreads) + threadIdx.x;
  u32x4 x0[kPackUnroll], x1[kPackUnroll];
  unsigned ochunk[kPackUnroll];   // output chunk over all slots (gi * per_slot + row chunk)
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    const unsigned idx = first + u * kThreads;
    ochunk[u] = total;
    if (idx < total) {
      unsigned gi, c, bt;
      if (fp8) {
        const unsigned ca = idx % cpr_all;
        bt = idx / cpr_all;
        gi = ca / cpr;
        c = ca - gi * cpr;
      } else {
        gi = idx / per_slot;
        const unsigned rem = idx - gi * per_slot;
        c = rem % cpr;
        bt = rem / cpr;
      }
      const unsigned t = bt % (unsigned)g.rows;
      const unsigned b = bt / (unsigned)g.rows;
      int p, srow;
      src_of_row(g, g.rank, (int)t, &p, &srow);
      const uint16_t* src = a.src[tensor][p] + (((size_t)b * g.shard_rows + srow) * H + hbase) * D +
                            (size_t)(gi * cpr + c) * elems_per_chunk;
      x0[u] = ld_stream<true>(src);
      if (fp8) x1[u] = ld_stream<true>(src + 8);
      ochunk[u] = gi * per_slot + bt * cpr + c;
    }
  }
  unsigned char* dst = (unsigned char*)a.dst[tensor];
#pragma unroll
  for (int u = 0; u < kPackUnroll; ++u) {
    if (ochunk[u] < total) {
      if (fp8) {
        u32x4 y;
        y.x = e4m3_of_bf16x4(x0[u].x, x0[u].y, inv);
        y.y = e4m3_of_bf16x4(x0[u].z, x0[u].w, inv);
        y.z = e4m3_of_bf16x4(x1[u].x, x1[u].y, inv);
        y.w = e4m3_of_bf16x4(x1[u].z, x1[u].w, inv);
        st_stream<false>(dst + (size_t)ochunk[u] * 16, y);
      } else {
        st_stream<true>(dst + (size_t)ochunk[u] * 16, x0[u]);
      }
    }
  }
}

// grid.x: chunks of one output shard's rows [B * shard_rows * ngroups * cpr] (as pack, the launch's heads
// of a row taken group after group, so consecutive lanes write one contiguous run of the shard row);
// grid.y = shard p.
__global__ __launch_bounds__(kThreads) void unpack_kernel(UnpackArgs a) {
  const RepackGeom& g = a.g;
  const int p = blockIdx.y;
  const int D = g.head_dim;
  const unsigned cpr = (unsigned)(a.gh * D / 8);
  const unsigned cpr_all = cpr * (unsigned)g.ngroups;
  const unsigned total = (unsigned)g.batch * (unsigned)g.shard_rows * cpr_all;
  const size_t slot_elems = (size_t)g.batch * g.rows * a.gh * D;
  const unsigned first = blockIdx.x * (kUnpackUnroll * kThreads) + threadIdx.x;
  u32x4 x[kUnpackUnroll];
  uint16_t* dst[kUnpackUnroll];
#pragma unroll
  for (int u = 0; u < kUnpackUnroll; ++u) {
    const unsigned idx = first + u * kThreads;
    dst[u] = nullptr;
    if (idx < total) {
      const unsigned ca = idx % cpr_all;
      const unsigned br = idx / cpr_all;
      const int r = (int)(br % (unsigned)g.shard_rows);      // row within shard p
      const unsigned b = br / (unsigned)g.shard_rows;
      const unsigned gi = ca / cpr, c = ca - gi * cpr;
      int t;
      if (g.rep_first) t = (r < g.n_rep) ? r : g.n_rep + p * g.s_local + (r - g.n_rep);
      else t = (r < g.s_local) ? p * g.s_local + r : g.degree * g.s_local + (r - g.s_local);
      x[u] = ld_stream<true>(a.src + gi * slot_elems + (((size_t)b * g.rows + t) * a.gh) * D + (size_t)c * 8);
      dst[u] = a.dst[p] + (((size_t)b * g.shard_rows + r) * a.heads + a.h0) * D + (size_t)ca * 8;
    }
  }
#pragma unroll
  for (int u = 0; u < kUnpackUnroll; ++u)
    if (dst[u] != nullptr) st_stream<false>(dst[u], x[u]);
}

__global__ void amax_zero_kernel(unsigned int* out) {
  if (threadIdx.x == 0) *out = 0u;
}

// |bf16| maximum of 8 elements as their 15 magnitude bits (finite inputs)
__device__ __forceinline__ unsigned int max_mag(u32x4 x, unsigned int m) {
  m = max(m, max(max(x.x & 0x7fffu, (x.x >> 16) & 0x7fffu), max(x.y & 0x7fffu, (x.y >> 16) & 0x7fffu)));
  return max(m, max(max(x.z & 0x7fffu, (x.z >> 16) & 0x7fffu), max(x.w & 0x7fffu, (x.w >> 16) & 0x7fffu)));
}

// grid: (blocks per tensor, tensors).  Each thread keeps kAmaxUnroll 16-byte loads in flight per round.
__global__ __launch_bounds__(kThreads) void amax_kernel(AmaxArgs a) {
  const u32x4* src = (const u32x4*)a.src[blockIdx.y];
  const size_t n = a.chunks_each;
  const size_t per_round = (size_t)gridDim.x * kThreads * kAmaxUnroll;
  unsigned int m = 0;
  for (size_t base = (size_t)blockIdx.x * kThreads * kAmaxUnroll + threadIdx.x; base < n; base += per_round) {
    u32x4 x[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const size_t i = base + (size_t)u * kThreads;
      x[u] = i < n ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = max_mag(x[u], m);
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
    const long total = (long)a.g[t].batch * a.g[t].rows * cpr * a.g[t].ngroups;
    if (total > most) most = total;
  }
  const long per_block = (long)kThreads * kPackUnroll;
  dim3 grid((unsigned)((most + per_block - 1) / per_block), 3);
  hipLaunchKernelGGL(pack_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_unpack(const UnpackArgs& a, hipStream_t s) {
  const long total = (long)a.g.batch * a.g.shard_rows * (a.gh * a.g.head_dim / 8) * a.g.ngroups;
  const long per_block = (long)kThreads * kUnpackUnroll;
  dim3 grid((unsigned)((total + per_block - 1) / per_block), a.g.degree);
  hipLaunchKernelGGL(unpack_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_amax(const AmaxArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(amax_zero_kernel, dim3(1), dim3(64), 0, s, a.out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // about kAmaxBlocks workgroups over all tensors, each keeping 8 chunks per thread in flight
  const size_t per_block = (size_t)kThreads * kAmaxUnroll;
  size_t blocks = (a.chunks_each + per_block - 1) / per_block;
  const size_t cap = (size_t)(kAmaxBlocks + a.n - 1) / a.n;
  if (blocks > cap) blocks = cap;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks, a.n), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace ulys
