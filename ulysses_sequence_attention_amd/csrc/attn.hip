// Dense non-causal attention with log-sum-exp for one head group, gfx950.
//
// What it computes (sglang layer.py LocalAttention / USPAttention.forward;
// flashdreams cp.py torch_sdpa_*): per (b, q head h, row i), over the keys J
// outside the batch's masked gap, s_ij = c <q_i, k_j>, o_i = softmax(s_i) V,
// lse_i = ln sum_J exp(s_ij); kv head = h / (hq / hkv) (GQA).
//
// How (MI355X-first):
//  * One workgroup = 256 query rows of one (b, h): 8 waves of 32 rows, two
//    waves per SIMD.  All waves share the K/V tiles in LDS.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    (or the fp8 v_mfma_scale_f32_32x32x64_f8f6f4 for e4m3 q/k): in the
//    accumulator every lane then holds ONE query row and 16 keys, so row max
//    and row sum are in-lane reductions plus one exchange with lane^32
//    (v_permlane32_swap), and the softmax probabilities are already laid out
//    as the B operand of the O^T = V^T P^T MFMA (no shuffles between the two
//    contractions).
//  * K and V tiles sit row-major in LDS (XOR-swizzled in 16- and 8-byte
//    chunks).  K fragments are plain 16-byte reads; V^T fragments come from
//    gfx950's transposing LDS read (ds_read_b64_tr_b16: within 16 lanes, four
//    8-byte row pieces are returned as columns), so V is never transposed in
//    registers or written element by element.
//  * 64-key tiles, double-buffered in LDS and filled by direct global->LDS
//    16-byte loads (no staging registers): the next tile streams in while
//    the current one is computed; one barrier per tile.
//  * Within a tile the two 32-key blocks are software-pipelined: the QK^T
//    MFMAs of block 1 are issued between the exp/convert instructions of
//    block 0, and the PV MFMAs of block 0 between the row-max instructions of
//    block 1, so each wave keeps its matrix core and vector ALU busy at once.
//  * Online softmax in the exp2 domain per 32-key block with a lazy max: the
//    running max is only raised (and O, l rescaled) when a block's max
//    exceeds it by more than 2^8, a wave-uniform branch; probabilities stay
//    <= 256, exact either way because the final normalisation divides by the
//    sum built with the same max.  Row sums are fp32 sums of the unrounded
//    probabilities (the LSE must not inherit the 2^-9 bf16 rounding of the
//    MFMA operand).
//  * Tiles wholly inside the key gap are skipped; the tail tile and tiles
//    that straddle the gap are masked per element.
// A head's arithmetic never depends on the other heads of the call, the grid
// or the slot strides, so a head-group split reproduces the full call's bytes.
#include "internal.h"

namespace ulys {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;             // query rows per workgroup
constexpr int kBN = 64;                      // keys per LDS tile (two 32-key blocks)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;                // raise the running max only past 2^8

template <int D, bool FP8>
struct Cfg {
  static constexpr int kQKBytes = FP8 ? 1 : 2;
  static constexpr int kKRow = D * kQKBytes;            // bytes per K row in LDS
  static constexpr int kKChunks = kKRow / 16;           // 16-byte chunks per K row
  static constexpr int kKSwz = kKChunks < 16 ? kKChunks : 16;
  static constexpr int kVRow = D * 2;                   // bytes per V row in LDS
  static constexpr int kVChunks = kVRow / 16;
  static constexpr int kKTile = kBN * kKRow;            // bytes
  static constexpr int kVTile = kBN * kVRow;            // bytes (bf16)
  static constexpr int kQKSteps = FP8 ? D / 64 : D / 16; // MFMAs along head_dim per 32x32 block
  static constexpr int kDB = D / 32;                     // 32-wide head_dim blocks of O
  static constexpr int kKSegs = kKTile / 1024;          // 1 KB LDS segments per tile
  static constexpr int kVSegs = kVTile / 1024;
  static constexpr int kKSegsPerWave = (kKSegs + kWaves - 1) / kWaves;
  static constexpr int kVSegsPerWave = (kVSegs + kWaves - 1) / kWaves;
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

template <int S>
struct StageTag { static constexpr int value = S; };

// 8-byte chunk index of V row `key` after the swizzle: rows read together by a
// transposing LDS read land on distinct banks.
template <int D>
__device__ __forceinline__ int vswz(int key, int chunk8) {
  return chunk8 ^ (D == 128 ? ((key & 3) << 3) : (((key >> 1) & 1) << 3));
}

__device__ __forceinline__ float lane_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

#define ULYS_INLINE __attribute__((always_inline))

template <int D, bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(AttnArgs a) {
  using C = Cfg<D, FP8>;
  // One LDS array per stage, selected at compile time: the compiler can then
  // prove that the DMA filling one stage never aliases reads of the other and
  // does not wait for in-flight tile loads before every LDS read.
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[C::kKTile];
  __shared__ __attribute__((aligned(16))) unsigned char k_lds1[C::kKTile];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[C::kVTile];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds1[C::kVTile];
  auto k_of = [&](auto st) -> unsigned char* { if constexpr (decltype(st)::value == 0) return k_lds0; else return k_lds1; };
  auto v_of = [&](auto st) -> unsigned char* { if constexpr (decltype(st)::value == 0) return v_lds0; else return v_lds1; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int qtile = blockIdx.x;
  const int head = blockIdx.y;
  const int b = blockIdx.z;
  const int rows = a.rows;
  const int kvh = head / (a.hq / a.hkv);

  float c = a.scale;
  if (FP8) {
    const float aq = a.amax[0], ak = a.amax[1];
    const float sq = aq > 0.0f ? __fdiv_rn(aq, 448.0f) : 1.0f;
    const float sk = ak > 0.0f ? __fdiv_rn(ak, 448.0f) : 1.0f;
    c = (c * sq) * sk;
  }
  const float c2 = c * kLog2e;

  // ---- key range: skip tiles wholly inside the gap ----
  const int ntiles = (rows + kBN - 1) / kBN;
  int gs = rows, ge = rows;   // empty gap
  if (a.has_gap) { gs = a.gap[b][0]; ge = a.gap[b][1]; if (ge <= gs) { gs = rows; ge = rows; } }
  const int skip_first = (gs + kBN - 1) / kBN;
  const int skip_last = (ge >= rows) ? ntiles : ge / kBN;   // tiles [skip_first, skip_last) are fully masked
  auto next_tile = [&](int j) {
    const int n = j + 1;
    return (n == skip_first && skip_last > n) ? skip_last : n;
  };
  const int first_tile = (skip_first == 0 && skip_last > 0) ? skip_last : 0;

  // ---- Q fragments in registers (B operand of S^T = K Q^T) ----
  const size_t q_row_stride = (size_t)a.hq * D;            // elements
  const size_t kv_row_stride = (size_t)a.hkv * D;
  const int qrow0 = qtile * kBM + wave * 32;
  constexpr int kQRegs = FP8 ? 8 : 4;                       // dwords per fragment
  unsigned int qf[C::kQKSteps][kQRegs];
  {
    const int row = qrow0 + l32;
    const unsigned char* qp = (const unsigned char*)a.q +
        (((size_t)b * rows + row) * q_row_stride + (size_t)head * D) * C::kQKBytes;
#pragma unroll
    for (int kk = 0; kk < C::kQKSteps; ++kk) {
      const int off = FP8 ? (kk * 64 + hh * 32) : (kk * 16 + hh * 8) * 2;   // bytes
#pragma unroll
      for (int part = 0; part < kQRegs / 4; ++part) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row < rows) x = ld16(qp + off + part * 16);
        qf[kk][part * 4 + 0] = x.x; qf[kk][part * 4 + 1] = x.y;
        qf[kk][part * 4 + 2] = x.z; qf[kk][part * 4 + 3] = x.w;
      }
    }
  }

  // ---- global -> LDS staging of one K/V tile (direct 16-byte loads) ----
  // global_load_lds_dwordx4 writes lane i's 16 bytes to LDS base + 16 i, so each
  // instruction fills one contiguous 1 KB segment; a lane picks the global chunk
  // that belongs at its LDS position under the XOR swizzle.  Rows past the end
  // are clamped to the last row (their scores are masked, their V is finite).
  const unsigned char* kbase = (const unsigned char*)a.k + ((size_t)b * rows * kv_row_stride + (size_t)kvh * D) * C::kQKBytes;
  const unsigned char* vbase = (const unsigned char*)a.v + ((size_t)b * rows * kv_row_stride + (size_t)kvh * D) * 2;
  auto load_tile = [&](int j, auto st) {
    unsigned char* kl = k_of(st);
    unsigned char* vl = v_of(st);
    const int k0 = j * kBN;
    constexpr int kKRowsPerSeg = 1024 / C::kKRow;
#pragma unroll
    for (int u = 0; u < C::kKSegsPerWave; ++u) {
      const int seg = wave + u * kWaves;
      if (C::kKSegs % kWaves != 0 && seg >= C::kKSegs) break;   // wave-uniform
      const int key = seg * kKRowsPerSeg + lane / C::kKChunks;
      const int sck = lane % C::kKChunks;
      const int ck = sck ^ (key & (C::kKSwz - 1));
      const int grow = min(k0 + key, rows - 1);
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(kbase + (size_t)grow * kv_row_stride * C::kQKBytes + ck * 16),
          (void __attribute__((address_space(3)))*)(&kl[seg * 1024]), 16, 0, 0);
    }
    constexpr int kVRowsPerSeg = 1024 / C::kVRow;
#pragma unroll
    for (int u = 0; u < C::kVSegsPerWave; ++u) {
      const int seg = wave + u * kWaves;
      if (C::kVSegs % kWaves != 0 && seg >= C::kVSegs) break;   // wave-uniform
      const int key = seg * kVRowsPerSeg + lane / C::kVChunks;
      const int sck = lane % C::kVChunks;                 // 16-byte slot in the LDS row
      const int ck = vswz<D>(key, 2 * sck) >> 1;          // its global 16-byte chunk
      const int grow = min(k0 + key, rows - 1);
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1)))*)(vbase + (size_t)grow * kv_row_stride * 2 + ck * 16),
          (void __attribute__((address_space(3)))*)(&vl[seg * 1024]), 16, 0, 0);
    }
  };

  // ---- running state ----
  f32x16 o[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m_run = -INFINITY;              // running max of c*log2e*s (lazy)
  float l_run0 = 0.0f, l_run1 = 0.0f;   // partial row sums (two chains)

  // End of a tile: this wave's tile loads have landed and its LDS reads are
  // done (s_waitcnt vmcnt(0) lgkmcnt(0), as a builtin so the compiler's own
  // wait tracking knows), then all waves meet at s_barrier.  The empty asm
  // statements keep the compiler from moving memory accesses across it.
  auto tile_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  load_tile(first_tile, StageTag<0>{});
  tile_barrier();

  // Per-lane LDS byte offsets of the MFMA operand reads, computed once: the
  // XOR swizzles only involve key bits that are the same for every 32-key
  // block, so each read is a base register plus a compile-time offset.
  //  K (A operand of S^T): lane row l32, head-dim chunk(s) of step kk.
  constexpr int kKOffs = FP8 ? 2 * C::kQKSteps : C::kQKSteps;
  int koff[kKOffs];
#pragma unroll
  for (int kk = 0; kk < C::kQKSteps; ++kk) {
    const int sw = l32 & (C::kKSwz - 1);
    if constexpr (!FP8) {
      koff[kk] = l32 * C::kKRow + (((kk * 2 + hh) ^ sw) * 16);
    } else {
      koff[2 * kk] = l32 * C::kKRow + (((kk * 4 + hh * 2) ^ sw) * 16);
      koff[2 * kk + 1] = l32 * C::kKRow + (((kk * 4 + hh * 2 + 1) ^ sw) * 16);
    }
  }
  //  V (A operand of O^T, transposing reads): within 16 lanes, lane 4j+t reads
  //  row key0 + j at head-dim d0 + 4t.. (see pv).
  const int g16 = lane >> 4, jrow = (lane >> 2) & 3, tcol = lane & 3;
  const int vkey0 = 4 * (g16 >> 1) + jrow;
  int voff[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
    voff[db] = vkey0 * C::kVRow + vswz<D>(vkey0, db * 8 + (g16 & 1) * 4 + tcol) * 8;

  // ---- block pieces ----
  // S^T for the 32 keys kb*32.. of the tile in K stage `kl`.
  auto qk = [&](const unsigned char* kl, int kb) ULYS_INLINE {
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
    const unsigned char* kblk = kl + kb * 32 * C::kKRow;
#pragma unroll
    for (int kk = 0; kk < C::kQKSteps; ++kk) {
      if constexpr (!FP8) {
        const u32x4 kx = *(const u32x4*)(kblk + koff[kk]);
        const u32x4 qx = {qf[kk][0], qf[kk][1], qf[kk][2], qf[kk][3]};
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kx), __builtin_bit_cast(bf16x8, qx), s,
                                                    0, 0, 0);
      } else {
        const u32x4 k0x = *(const u32x4*)(kblk + koff[2 * kk]);
        const u32x4 k1x = *(const u32x4*)(kblk + koff[2 * kk + 1]);
        const i32x8 af = {(int)k0x.x, (int)k0x.y, (int)k0x.z, (int)k0x.w,
                          (int)k1x.x, (int)k1x.y, (int)k1x.z, (int)k1x.w};
        const i32x8 bq = {(int)qf[kk][0], (int)qf[kk][1], (int)qf[kk][2], (int)qf[kk][3],
                          (int)qf[kk][4], (int)qf[kk][5], (int)qf[kk][6], (int)qf[kk][7]};
        s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bq, s, 0, 0, 0, 127, 0, 127);
      }
    }
    return s;
  };

  // Tail keys and keys inside the gap -> -inf: branch-free selects under one
  // wave-uniform branch (the key of register r is kb0 + 8 (r/4) + 4 hh + r%4).
  auto mask = [&](f32x16& s, int kb0) ULYS_INLINE {
    if (kb0 + 32 > rows || (kb0 < ge && kb0 + 32 > gs)) {
      const int kl = kb0 + 4 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kidx = kl + 8 * (r >> 2) + (r & 3);
        const bool dead = (kidx >= rows) | ((kidx >= gs) & (kidx < ge));
        s[r] = dead ? -INFINITY : s[r];
      }
    }
  };

  // Row max of a block, in the exp2 domain.
  auto rowmax = [&](const f32x16& s) ULYS_INLINE {
    float m = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, s[r]);
    return lane_swap_max(m) * c2;
  };

  // Lazy rescale before a block's probabilities are formed.
  auto rescale = [&](float mx) ULYS_INLINE {
    if (__any(mx > m_run + kLazy)) {
      const float mn = fmaxf(m_run, mx);
      const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      l_run0 *= alpha;
      l_run1 *= alpha;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
  };

  // Probabilities -> bf16 B operands of the PV MFMA (p[e] = accumulator
  // registers 8e..8e+7) and fp32 row sums.
  auto probs = [&](const f32x16& s, bf16x8 (&p)[2]) ULYS_INLINE {
    const float mb = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * e + 2 * i], c2, -mb));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * e + 2 * i + 1], c2, -mb));
        const f32x2 xx = {x0, x1};
        const bf16x2 pk = __builtin_convertvector(xx, bf16x2);
        p[e][2 * i] = pk[0];
        p[e][2 * i + 1] = pk[1];
        l_run0 += x0;
        l_run1 += x1;
      }
  };

  // The probabilities and row sums are complete here (the empty asm consumes
  // them), so the compiler schedules their VALU work between the QK^T MFMAs
  // issued before this point instead of sinking it past the mask branch.
  auto pin = [&](const bf16x8 (&pp)[2]) ULYS_INLINE {
    asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pp[0])), "v"(__builtin_bit_cast(u32x4, pp[1])), "v"(l_run0),
                 "v"(l_run1));
  };

  // O^T += V^T P^T for the 32 keys kb*32.. of the tile in V stage `vl`.  A
  // operand of lane l: V[key(hh, i)][d = 32 db + l%32], i = 0..7, read as two
  // transposing 8-byte loads over keys base + 4 hh + (0..3) and
  // base + 8 + 4 hh + (0..3) -- the keys whose probabilities p[e] holds.
  auto pv = [&](const unsigned char* vl, int kb, const bf16x8 (&p)[2]) ULYS_INLINE {
#pragma unroll
    for (int db = 0; db < C::kDB; ++db) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const unsigned char* va_p = vl + (kb * 32 + 16 * e) * C::kVRow + voff[db];
        const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(unsigned char*)(va_p));
        const bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(unsigned char*)(va_p + 8 * C::kVRow));
        const bf16x8 af = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, p[e], o[db], 0, 0, 0);
      }
    }
  };

  // One tile, software-pipelined over its two blocks:
  //   QK 0, mask/max/rescale 0 | {QK 1 + probabilities 0} | mask 1 |
  //   {PV 0 + row max 1} | rescale 1, probabilities 1, PV 1.
  auto compute_tile = [&](int j, auto st) {
    const unsigned char* kl = k_of(st);
    const unsigned char* vl = v_of(st);
    const int k0 = j * kBN;
    bf16x8 p[2];
    f32x16 s0 = qk(kl, 0);
    mask(s0, k0);
    rescale(rowmax(s0));
    f32x16 s1 = qk(kl, 1);
    probs(s0, p);
    pin(p);
    mask(s1, k0 + 32);
    pv(vl, 0, p);
    const float m1 = rowmax(s1);
    rescale(m1);
    probs(s1, p);
    pv(vl, 1, p);
  };

  // Tiles alternate between the two stages; the next tile's loads are issued
  // before the current tile is computed.
  for (int j = first_tile;;) {
    int jn = next_tile(j);
    if (jn < ntiles) load_tile(jn, StageTag<1>{});
    compute_tile(j, StageTag<0>{});
    tile_barrier();
    if (jn >= ntiles) break;
    j = jn;
    jn = next_tile(j);
    if (jn < ntiles) load_tile(jn, StageTag<0>{});
    compute_tile(j, StageTag<1>{});
    tile_barrier();
    if (jn >= ntiles) break;
    j = jn;
  }

  // ---- epilogue: normalise, write o (bf16) and lse (fp32, natural log) ----
  {
    const int row = qrow0 + l32;
    const float l = lane_swap_sum(l_run0 + l_run1);
    const float inv = 1.0f / l;
    if (row < rows) {
      uint16_t* op = a.o + ((size_t)b * rows + row) * q_row_stride + (size_t)head * D;
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x2 lo = {o[db][4 * r4 + 0] * inv, o[db][4 * r4 + 1] * inv};
          const f32x2 hi = {o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv};
          const bf16x2 blo = __builtin_convertvector(lo, bf16x2);
          const bf16x2 bhi = __builtin_convertvector(hi, bf16x2);
          u32x2 w;
          w.x = __builtin_bit_cast(unsigned int, blo);
          w.y = __builtin_bit_cast(unsigned int, bhi);
          *(u32x2*)(op + db * 32 + 8 * r4 + 4 * hh) = w;
        }
      if (a.lse != nullptr && hh == 0)
        a.lse[((size_t)b * a.hq + head) * rows + row] = (m_run + __log2f(l)) * kLn2;
    }
  }
}

template <int D, bool FP8>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.rows + kBM - 1) / kBM, a.hq, a.batch);
  hipLaunchKernelGGL((attn_fwd_kernel<D, FP8>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, int head_dim, bool fp8, hipStream_t s) {
  if (head_dim == 128) return fp8 ? launch<128, true>(a, s) : launch<128, false>(a, s);
  return fp8 ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace ulys
