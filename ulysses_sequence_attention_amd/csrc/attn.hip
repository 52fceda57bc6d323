// Dense non-causal attention with log-sum-exp for one head group, gfx950.
//
// What it computes (sglang layer.py LocalAttention / USPAttention.forward;
// flashdreams cp.py torch_sdpa_*): per (b, q head h, row i), over the keys J
// outside the batch's masked gap, s_ij = c <q_i, k_j>, o_i = softmax(s_i) V,
// lse_i = ln sum_J exp(s_ij); kv head = h / (hq / hkv) (GQA).
//
// How (MI355X-first):
//  * One workgroup = 256 query rows of one (b, h); all its waves share the K/V
//    tiles in LDS.  Two wave shapes (NH = row halves per wave):
//     - bf16 q/k, head_dim 128, no key mask (NH = 2): 4 waves of 64 rows, one
//       wave per SIMD.  Every K and V fragment read from LDS feeds the MFMAs of
//       both 32-row halves, which halves the LDS bytes per MFMA.  O (128 regs)
//       and Q (64) live in AGPRs, so the two contractions are inline-asm MFMAs
//       (AGPR accumulator for PV, AGPR B operand for QK^T), and the loop body
//       is placed by hand: one MFMA per issue group with one probability
//       element beside it (scaled score, exponential, sum-and-pack three
//       groups deep), an LDS read or a tile load beside every other one.  The
//       compiler sees neither these MFMAs' latency nor their operands'
//       hazards, so the waits are placed here: an MFMA result is read by VALU
//       no sooner than 12 wait states after the MFMA (the count the compiler
//       itself inserts on gfx950), and an operand written by VALU is read by an
//       MFMA no sooner than 2 wait states after the write.
//     - otherwise (fp8 q/k, head_dim 64, a key mask; NH = 1): 8 waves of 32
//       rows, two waves per SIMD, builtin MFMAs.
//    Both shapes do the same arithmetic per row in the same order, so their
//    outputs are bit-identical.
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
//  * 64-key tiles in a three-stage LDS ring, filled by direct global->LDS
//    16-byte loads (no staging registers) two tiles ahead; one barrier per
//    tile.
//  * Software pipeline over 32-key blocks: while block b's probabilities are
//    formed (VALU), the wave issues the PV MFMAs of block b-1 and the QK^T
//    MFMAs of block b+1, which do not depend on them; K operands of b+1 and V
//    operands of b are read from LDS one phase before their MFMAs.  With one
//    wave per SIMD the clean steps also spread their tile loads over the PV
//    MFMAs of their first block instead of issuing them in one burst.
//  * Online softmax in the exp2 domain per 32-key block with a lazy max: the
//    probabilities of a block are formed speculatively with the current
//    running max, and the max is only raised (O, l rescaled, the block's
//    scores recomputed from K in LDS and its probabilities redone) when a
//    lane's sum of its 16 probabilities exceeds 2^8 -- which any probability
//    above 2^8 causes, and which bounds every probability by 2^8 otherwise --
//    or while the row has no finite max yet.  A wave-uniform branch taken a
//    few times per row, checked after the MFMAs; no per-block max.  Exact
//    either way, because the final normalisation divides by the sum built
//    with the same max.  Row sums are fp32 sums of the unrounded
//    probabilities (the LSE must not inherit the 2^-9 bf16 rounding of the
//    MFMA operand).
//  * Tiles wholly inside the key gap are skipped; the tail tile and tiles
//    that straddle the gap are masked per element.
//  * Steps over clean tiles (no key past the end or in the gap, and with a
//    key mask, runs of consecutive listed tiles whose keys are all valid) run
//    in whole ring rounds with the stages compile-time constants: every LDS
//    read and tile-load address is then a register plus an immediate, with no
//    address arithmetic in the step.
//  * Under a range split the workgroups are ordered so that each XCD takes a
//    contiguous block of (range, head) indices, sharing a head's K/V in its
//    L2.
//  * Work per workgroup: one query tile over all its key tiles; or, under a
//    key-range split, a contiguous run of them; or, under a range split, a
//    run of its (b, h)'s (query tile, key tile) sequence, walked as pieces.
//    A tile computed in parts leaves fp32 partials (o, lse) that a second
//    kernel merges in a fixed order (split_merge_kernel, range_merge_kernel).
//  * Output rows (bf16, or the fp32 partials) leave through a per-wave LDS
//    staging area, 128 bytes of each row at a time, so that every global
//    store writes whole 128-byte lines.
// A head's arithmetic never depends on the other heads of the call, the grid
// or the slot strides, so a head-group split reproduces the full call's bytes.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "internal.h"

namespace ulys {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;             // query rows per workgroup
constexpr int kBN = kAttnKeysPerTile;        // keys per LDS tile (two 32-key blocks)
constexpr int kStages = 3;                   // LDS ring depth (tiles)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazySum = 256.0f;           // raise the running max when a lane's block sum exceeds 2^8

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
};

// Row halves of 32 query rows per wave: two (one wave per SIMD, O and Q in
// AGPRs) for bf16 q/k at head_dim 128 without a key mask, else one.
template <int D, bool FP8, bool MASK>
constexpr int kRowHalves = (D == 128 && !FP8 && !MASK) ? 2 : 1;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }

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

// One 16-byte-per-lane global->LDS load (global_load_lds_dwordx4: lane i's 16
// bytes land at LDS m0 + 16 i).  Issued as inline asm so that the compiler does
// not treat it as an LDS store it must wait for before unrelated LDS reads of
// other ring stages; the kernel waits for these loads itself (vmcnt) before the
// barrier that publishes a tile.  m0 is set here and used by nothing else.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The global address is a scalar base plus a 32-bit per-lane offset, so a
// load needs no vector address arithmetic.
__device__ __forceinline__ void dma16(const void* sbase, unsigned int voff, unsigned int lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ unsigned int lds_u32(const void* p) {
  return (unsigned int)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

template <int D, bool FP8, bool MASK, int NH>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads / NH, kThreads / NH), amdgpu_waves_per_eu(3 - NH, 3 - NH)))
void attn_fwd_kernel(AttnArgs a) {
  using C = Cfg<D, FP8>;
  static_assert(NH == kRowHalves<D, FP8, MASK>, "wave shape");
  // NH row halves of 32 query rows per wave, kW waves per workgroup (kBM rows)
  constexpr int kW = kWaves / NH;
  constexpr int kT = kW * 64;
  constexpr int kKSegsPerWave = (C::kKSegs + kW - 1) / kW;   // 1 KB tile-load segments per wave
  constexpr int kVSegsPerWave = (C::kVSegs + kW - 1) / kW;
  constexpr int kLoadsPerTile = kKSegsPerWave + kVSegsPerWave;
  // One LDS array per stage, selected at compile time: the compiler can then
  // prove that the DMA filling one stage never aliases reads of the other and
  // does not wait for in-flight tile loads before every LDS read.
  // The LDS ring: three stages of one K tile and one V tile each.
  __shared__ __attribute__((aligned(16))) unsigned char lds[kStages * (C::kKTile + C::kVTile)];
  // Tiles with at least one valid key, in order, when a key mask is given.
  __shared__ unsigned short tile_list[kMaxMaskTiles];
  static_assert(kMaxMaskTiles <= 0x1000, "tile index in the low 12 bits of a tile-list entry");
  // Per-wave staging of the output rows (128 bytes of each row at a time, rows
  // 144 bytes apart): global stores then write whole lines.
  constexpr int kStgPitch = 144;
  __shared__ __attribute__((aligned(16))) unsigned char stage_lds[kWaves * 32 * kStgPitch];
  // Stage st's K tile; its V tile sits at v_of(st) + the V region offset, which
  // the per-lane V read offsets carry (so every LDS read's immediate offset
  // stays below 64 KB).
  auto k_of = [&](auto st) -> unsigned char* { return lds + int(st) * C::kKTile; };
  auto v_of = [&](auto st) -> unsigned char* { return lds + int(st) * C::kVTile; };
  constexpr int kVRegion = kStages * C::kKTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // This workgroup's work: with a range split (a.ranges > 0), range wx of its
  // (b, head)'s (query tile, key tile) sequence; otherwise query tile qtile0,
  // key-range chunk `split` of a.splits.
  const bool ranged = a.ranges > 0;
  // Under a range split, workgroup w of the launch runs on XCD w % 8; when the
  // workgroups divide evenly, XCD x takes the x-th contiguous block of (range,
  // head, batch) indices, so the workgroups of one XCD walk neighbouring ranges
  // of one head and share its K/V tiles in that XCD's L2 (measured +1%).
  int wx = blockIdx.x, wy = blockIdx.y, wz = blockIdx.z;
  if (ranged) {
    const unsigned nwg = gridDim.x * gridDim.y * gridDim.z;
    if ((nwg & 7u) == 0) {
      const unsigned w = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
      const unsigned w2 = (w & 7u) * (nwg >> 3) + (w >> 3);
      const unsigned rest = w2 / gridDim.x;
      wx = __builtin_amdgcn_readfirstlane((int)(w2 - rest * gridDim.x));
      wy = __builtin_amdgcn_readfirstlane((int)(rest % gridDim.y));
      wz = __builtin_amdgcn_readfirstlane((int)(rest / gridDim.y));
    }
  }
  const int split = ranged ? 0 : wx / a.qtiles;
  const int qtile0 = ranged ? 0 : wx - split * a.qtiles;
  const int hl = wy;                  // head within this launch
  const int head = a.head0 + hl;
  const int b = wz;
  const int qrows = a.q_rows;
  const int rows = a.kv_rows;   // keys
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

  // ---- Q fragments in registers (B operand of S^T = K Q^T) ----
  const size_t q_row_stride = (size_t)a.hq * D;            // elements
  const size_t kv_row_stride = (size_t)a.hkv * D;
  constexpr int kQRegs = FP8 ? 8 : 4;                       // dwords per fragment
  unsigned int qf[NH][C::kQKSteps][kQRegs];
  u32x4 qa[NH][C::kQKSteps];   // two row halves: Q operands as whole AGPR tuples
  // The thread index as a value the compiler cannot see through: per-lane
  // addresses of the per-piece work (Q loads, output writes, merge) are
  // formed from it inside the piece loop instead of being hoisted out of it
  // and held in registers across the key loop.
  auto fresh_tid = [&]() {
    int t;
    asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(tid));
    return t;
  };
  auto load_q = [&](int qrow0) {
    const int ft = fresh_tid();
#pragma unroll
    for (int rh = 0; rh < NH; ++rh) {
    const int row = qrow0 + rh * 32 + (ft & 31), hh = (ft >> 5) & 1;
    const unsigned char* qp = (const unsigned char*)a.q +
        (((size_t)b * qrows + row) * q_row_stride + (size_t)head * D) * C::kQKBytes;
#pragma unroll
    for (int kk = 0; kk < C::kQKSteps; ++kk) {
      const int off = FP8 ? (kk * 64 + hh * 32) : (kk * 16 + hh * 8) * 2;   // bytes
#pragma unroll
      for (int part = 0; part < kQRegs / 4; ++part) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row < qrows) x = ld16(qp + off + part * 16);
        if constexpr (NH == 2) {
          // copied into an AGPR tuple once per piece; the wait states cover the
          // write before the first QK^T MFMA reads it
          asm volatile("s_nop 4" : "=a"(qa[rh][kk]) : "0"(x));
        } else {
        qf[rh][kk][part * 4 + 0] = x.x; qf[rh][kk][part * 4 + 1] = x.y;
        qf[rh][kk][part * 4 + 2] = x.z; qf[rh][kk][part * 4 + 3] = x.w;
        }
      }
    }
    }
  };

  // ---- global -> LDS staging of one K/V tile (direct 16-byte loads) ----
  // global_load_lds_dwordx4 writes lane i's 16 bytes to LDS base + 16 i, so each
  // instruction fills one contiguous 1 KB segment; a lane picks the global chunk
  // that belongs at its LDS position under the XOR swizzle.  The tile's first
  // row is a scalar base and each lane's byte offset from it is computed once;
  // in the last tile, when the keys end inside it, rows past the end are
  // clamped to the last row (their scores are masked, their V is finite) by
  // offsets of its own.
  const unsigned char* kbase = (const unsigned char*)a.k + ((size_t)b * rows * kv_row_stride + (size_t)kvh * D) * C::kQKBytes;
  const unsigned char* vbase = (const unsigned char*)a.v + ((size_t)b * rows * kv_row_stride + (size_t)kvh * D) * 2;
  const unsigned int krow = (unsigned int)(kv_row_stride * C::kQKBytes);   // bytes per key row
  const unsigned int vrow = (unsigned int)(kv_row_stride * 2);
  const int last_rows = rows - (ntiles - 1) * kBN;                       // keys in the last tile
  constexpr int kKRowsPerSeg = 1024 / C::kKRow;
  constexpr int kVRowsPerSeg = 1024 / C::kVRow;
  // A wave's u-th load of a tile fetches segment wave + 8u: the same lanes at
  // 8 kRowsPerSeg more rows (a multiple of the swizzle period), so only its
  // first offset is per lane and the others move the scalar base.  With fewer
  // segments than waves (one load each), a surplus wave repeats the last
  // segment, which keeps every wave's load count per tile the same.
  static_assert(kKSegsPerWave == 1 || C::kKSegs % kW == 0, "whole segments per wave");
  static_assert(kVSegsPerWave == 1 || C::kVSegs % kW == 0, "whole segments per wave");
  static_assert((kW * kKRowsPerSeg) % C::kKSwz == 0 && (kW * kVRowsPerSeg) % 4 == 0, "swizzle period");
  const int kseg = min(wave, C::kKSegs - 1), vseg = min(wave, C::kVSegs - 1);
  const int kkey = kseg * kKRowsPerSeg + lane / C::kKChunks;
  const int kck = (lane % C::kKChunks) ^ (kkey & (C::kKSwz - 1));
  const unsigned int kgo = kkey * krow + kck * 16;
  const unsigned int kls = __builtin_amdgcn_readfirstlane(kseg * 1024);
  const int vkey = vseg * kVRowsPerSeg + lane / C::kVChunks;
  const int vck = vswz<D>(vkey, 2 * (lane % C::kVChunks)) >> 1;   // global 16-byte chunk of this LDS slot
  const unsigned int vgo = vkey * vrow + vck * 16;
  const unsigned int vls = __builtin_amdgcn_readfirstlane(vseg * 1024);
  const unsigned int ktile = kBN * krow, vtile = kBN * vrow;   // bytes per tile (hq <= 65535: fits)
  const int tail_tile = last_rows < kBN ? ntiles - 1 : -1;
  unsigned int kgo_u[kKSegsPerWave], vgo_u[kVSegsPerWave];
#pragma unroll
  for (int u = 0; u < kKSegsPerWave; ++u) kgo_u[u] = kgo + u * kW * kKRowsPerSeg * krow;
#pragma unroll
  for (int u = 0; u < kVSegsPerWave; ++u) vgo_u[u] = vgo + u * kW * kVRowsPerSeg * vrow;
  auto load_tile = [&](int j, auto st) {
    const unsigned int kl = lds_u32(k_of(st)) + kls;
    const unsigned int vl = lds_u32(v_of(st) + kVRegion) + vls;
    const unsigned char* kt = kbase + (size_t)(unsigned int)j * ktile;
    const unsigned char* vt = vbase + (size_t)(unsigned int)j * vtile;
    if (j == tail_tile) {
      // The last tile, when the keys end inside it: rows past the end are
      // clamped to the last row (their scores are masked, their V is finite).
      // (lane index laundered so this stays inside the rarely taken branch)
      int ln;
      asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
      const int kr = kseg * kKRowsPerSeg + ln / C::kKChunks, vr = vseg * kVRowsPerSeg + ln / C::kVChunks;
      const unsigned int kc = ((ln % C::kKChunks) ^ (kr & (C::kKSwz - 1))) * 16;
      const unsigned int vc = (vswz<D>(vr, 2 * (ln % C::kVChunks)) >> 1) * 16;
#pragma unroll
      for (int u = 0; u < kKSegsPerWave; ++u)
        dma16(kt, min(kr + u * kW * kKRowsPerSeg, last_rows - 1) * krow + kc, kl + u * kW * 1024);
#pragma unroll
      for (int u = 0; u < kVSegsPerWave; ++u)
        dma16(vt, min(vr + u * kW * kVRowsPerSeg, last_rows - 1) * vrow + vc, vl + u * kW * 1024);
    } else {
#pragma unroll
      for (int u = 0; u < kKSegsPerWave; ++u) dma16(kt, kgo_u[u], kl + u * kW * 1024);
#pragma unroll
      for (int u = 0; u < kVSegsPerWave; ++u) dma16(vt, vgo_u[u], vl + u * kW * 1024);
    }
  };

  // ---- running state ----
  // (set by reset_state at the start of every piece of work)
  f32x16 o[NH][C::kDB];
  float m_run[NH];   // running max of c*log2e*s (lazy)
  float negm[NH];    // -m_run, or 0 while m_run is -inf
  // A block raises m_run when this lane's sum of its 16 probabilities exceeds
  // thr: 2^8 (probabilities are >= 0, so a sum <= 2^8 bounds each of them by
  // 2^8, and a probability above 2^8 makes the sum exceed it), or -1 while
  // m_run is -inf (every block raises until the row has a finite max).
  float thr[NH];
  float l_run[NH];   // row sum (this lane's half of the keys)
  // Two row halves (O in AGPRs, written by asm MFMAs whose latency the
  // compiler cannot see): 24 wait states before VALU reads O (rescale,
  // epilogue), tied to O so that no read of it moves above them; and 4 after
  // VALU writes it (zeroing, rescale) before the next asm MFMA reads it.
  static_assert(NH == 1 || C::kDB == 4, "two row halves at head_dim 128");
  auto settle_o = [&](int rh) ULYS_INLINE {
    if constexpr (NH == 2) {
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[rh][0]), "+a"(o[rh][1]), "+a"(o[rh][2]), "+a"(o[rh][3]));
    }
  };
  auto settle_o_written = [&](int rh) ULYS_INLINE {
    if constexpr (NH == 2) {
      asm volatile("s_nop 3" : "+a"(o[rh][0]), "+a"(o[rh][1]), "+a"(o[rh][2]), "+a"(o[rh][3]));
    }
  };
  auto reset_state = [&]() {
#pragma unroll
    for (int rh = 0; rh < NH; ++rh) {
#pragma unroll
      for (int db = 0; db < C::kDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[rh][db][r] = 0.0f;
      settle_o_written(rh);
      m_run[rh] = -INFINITY;
      negm[rh] = 0.0f;
      thr[rh] = -1.0f;
      l_run[rh] = 0.0f;
    }
  };

  // Barrier publishing the next tile: this wave's loads of that tile have
  // landed (s_waitcnt vmcnt(N): at most the later tiles' loads still in flight;
  // an immediate, so the count per tile is uniform across waves), then all
  // waves meet at s_barrier.  LDS reads still in flight are of stages in use
  // and may cross it.  The empty asm statements keep the compiler from moving
  // memory accesses across it.
  constexpr int kInFlight = (kStages - 3) * kLoadsPerTile;
  static_assert(kInFlight < 16, "vmcnt immediate");
  auto tile_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70 | kInFlight);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Per-lane LDS byte offsets of the MFMA operand reads, computed once: the
  // XOR swizzles only involve key bits that are the same for every 32-key
  // block, so each read is a base register plus a compile-time offset.
  //  K (A operand of S^T): lane row l32, head-dim chunk(s) of step kk, in the
  //  stage the key loop reads next (stage 1 for the first step).  kcur moves
  //  by one stage per step, so in the loop a K read is this register plus a
  //  compile-time offset; other stages are reached by a scalar delta.
  constexpr int kKOffs = FP8 ? 2 * C::kQKSteps : C::kQKSteps;
  int kcur[kKOffs];
  auto reset_kcur = [&]() {
#pragma unroll
    for (int kk = 0; kk < C::kQKSteps; ++kk) {
      const int sw = l32 & (C::kKSwz - 1);
      if constexpr (!FP8) {
        kcur[kk] = C::kKTile + l32 * C::kKRow + (((kk * 2 + hh) ^ sw) * 16);
      } else {
        kcur[2 * kk] = C::kKTile + l32 * C::kKRow + (((kk * 4 + hh * 2) ^ sw) * 16);
        kcur[2 * kk + 1] = C::kKTile + l32 * C::kKRow + (((kk * 4 + hh * 2 + 1) ^ sw) * 16);
      }
    }
  };
  //  V (A operand of O^T, transposing reads): within 16 lanes, lane 4j+t reads
  //  row key0 + j at head-dim d0 + 4t.. (see read_v).
  const int g16 = lane >> 4, jrow = (lane >> 2) & 3, tcol = lane & 3;
  const int vkey0 = 4 * (g16 >> 1) + jrow;
  int voff[C::kDB];
#pragma unroll
  for (int db = 0; db < C::kDB; ++db)
    voff[db] = kVRegion + vkey0 * C::kVRow + vswz<D>(vkey0, db * 8 + (g16 & 1) * 4 + tcol) * 8;
#pragma unroll
  for (int db = 0; db < C::kDB; ++db) asm volatile("" : "+v"(voff[db]));   // keep the region offset in the register

  // ---- block pieces ----
  struct KFrag { u32x4 x[kKOffs]; };      // K operands of one 32-key block
  struct VFrag { bf16x8 x[C::kDB][2]; };  // V^T operands of one 32-key block

  // K operands of block kb of the stage `delta` bytes from kcur's (one, or all).
  auto read_k_one = [&](int delta, auto kb, int i, KFrag& kf) ULYS_INLINE {
    kf.x[i] = *(const u32x4*)(lds + kcur[i] + delta + int(kb) * 32 * C::kKRow);
  };
  auto read_k = [&](int delta, auto kb, KFrag& kf) ULYS_INLINE {
#pragma unroll
    for (int i = 0; i < kKOffs; ++i) read_k_one(delta, kb, i, kf);
  };

  // One head-dim step kk of S^T = K Q^T (row half rh).  Two row halves: an
  // inline-asm MFMA reading Q from its AGPR tuple (a builtin would pull Q into
  // VGPRs); the first step writes a fresh accumulator, early-clobbered so that
  // it shares no register with the K operand.  Its result is read by VALU only
  // after the wait states of the caller.
  auto qk_step = [&](const KFrag& kf, int kk, f32x16 s, int rh) ULYS_INLINE {
    if constexpr (NH == 2) {
      const u32x4 qx = qa[rh][kk];
      if (kk == 0)
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(kf.x[kk]), "a"(qx));
      else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(kf.x[kk]), "a"(qx));
      return s;
    } else if constexpr (!FP8) {
      const u32x4 qx = {qf[rh][kk][0], qf[rh][kk][1], qf[rh][kk][2], qf[rh][kk][3]};
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf.x[kk]),
                                                     __builtin_bit_cast(bf16x8, qx), s, 0, 0, 0);
    } else {
      const u32x4 k0x = kf.x[2 * kk], k1x = kf.x[2 * kk + 1];
      const i32x8 af = {(int)k0x.x, (int)k0x.y, (int)k0x.z, (int)k0x.w,
                        (int)k1x.x, (int)k1x.y, (int)k1x.z, (int)k1x.w};
      const i32x8 bq = {(int)qf[rh][kk][0], (int)qf[rh][kk][1], (int)qf[rh][kk][2], (int)qf[rh][kk][3],
                        (int)qf[rh][kk][4], (int)qf[rh][kk][5], (int)qf[rh][kk][6], (int)qf[rh][kk][7]};
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bq, s, 0, 0, 0, 127, 0, 127);
    }
  };
  // S^T = K Q^T for one 32-key block (row half rh).  Two row halves: 20 wait
  // states before any VALU read of the scores.
  auto qk = [&](const KFrag& kf, int rh) ULYS_INLINE {
    f32x16 s;
    if constexpr (NH == 2) {
#pragma unroll
      for (int kk = 0; kk < C::kQKSteps; ++kk) s = qk_step(kf, kk, s, rh);
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(s));
      return s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < C::kQKSteps; ++kk) {
      if constexpr (!FP8) {
        const u32x4 qx = {qf[rh][kk][0], qf[rh][kk][1], qf[rh][kk][2], qf[rh][kk][3]};
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf.x[kk]),
                                                    __builtin_bit_cast(bf16x8, qx), s, 0, 0, 0);
      } else {
        const u32x4 k0x = kf.x[2 * kk], k1x = kf.x[2 * kk + 1];
        const i32x8 af = {(int)k0x.x, (int)k0x.y, (int)k0x.z, (int)k0x.w,
                          (int)k1x.x, (int)k1x.y, (int)k1x.z, (int)k1x.w};
        const i32x8 bq = {(int)qf[rh][kk][0], (int)qf[rh][kk][1], (int)qf[rh][kk][2], (int)qf[rh][kk][3],
                          (int)qf[rh][kk][4], (int)qf[rh][kk][5], (int)qf[rh][kk][6], (int)qf[rh][kk][7]};
        s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af, bq, s, 0, 0, 0, 127, 0, 127);
      }
    }
    return s;
  };

  // V^T operands of one 32-key block: lane l needs V[key(hh, i)][d = 32 db + l%32],
  // i = 0..7, read as two transposing 8-byte loads over keys base + 4 hh + (0..3)
  // and base + 8 + 4 hh + (0..3) -- the keys whose probabilities p[e] holds.
  auto read_v_one = [&](const unsigned char* vl, auto kb, int db, int e, VFrag& vf) ULYS_INLINE {
    const unsigned char* va_p = vl + (int(kb) * 32 + 16 * e) * C::kVRow + voff[db];
    const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4*)(unsigned char*)(va_p));
    const bf16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4*)(unsigned char*)(va_p + 8 * C::kVRow));
    vf.x[db][e] = __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto read_v = [&](const unsigned char* vl, auto kb, VFrag& vf) ULYS_INLINE {
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e) read_v_one(vl, kb, db, e, vf);
  };

  // One PV MFMA.  With two row halves O lives in AGPRs: the accumulate is
  // written as inline asm with an AGPR accumulator (the VGPR form of the
  // builtin would need all of O in VGPRs).  Its P operand is written by VALU at
  // least 2 wait states earlier: a block before, or after the wait states that
  // end the max-raise path and the piece set-up.
  auto pv_one = [&](f32x16& acc, const bf16x8& va, const bf16x8& pb) ULYS_INLINE {
    if constexpr (NH == 2) {
      asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(va), "v"(pb));
    } else {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc, 0, 0, 0);
    }
  };
  // O^T += V^T P^T for one 32-key block.
  auto pv = [&](const VFrag& vf, const bf16x8 (&p)[NH][2]) ULYS_INLINE {
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int rh = 0; rh < NH; ++rh) pv_one(o[rh][db], vf.x[db][e], p[rh][e]);
  };

  // Valid-key bits of the 32 keys from kb0 (bit j: key kb0 + j): inside
  // [0, rows), outside the gap, and set in the key mask when one is given.
  // (MASK: the launch was given a key mask; without one, none of the mask code is compiled in)
  const uint32_t* mask_row = MASK ? a.key_mask + (size_t)b * a.mask_words : nullptr;
  auto bits_in = [](int k0, int lo, int hi) -> unsigned {
    const int x = min(max(lo - k0, 0), 32), y = min(max(hi - k0, 0), 32);
    if (y <= x) return 0u;
    const unsigned below_y = y == 32 ? ~0u : ((1u << y) - 1u);
    const unsigned below_x = x == 32 ? ~0u : ((1u << x) - 1u);
    return below_y & ~below_x;
  };
  auto mask_word = [&](int kb0) -> unsigned {   // a load issued a block ahead of its use, or all valid
    if constexpr (MASK) return kb0 < rows ? mask_row[kb0 >> 5] : 0u;
    else return ~0u;
  };
  auto straddles = [&](int kb0) { return kb0 + 32 > rows || (kb0 < ge && kb0 + 32 > gs); };
  auto valid_bits = [&](int kb0, unsigned mword) -> unsigned {
    unsigned v = mword;
    if (straddles(kb0)) v &= bits_in(kb0, 0, rows) & ~bits_in(kb0, gs, ge);
    return v;
  };

  // Invalid keys of the block from kb0 -> -inf: selects under one wave-uniform
  // branch, taken for blocks that straddle the end or the gap, or whose mask
  // word (uniform, scalar) is not all ones (the key of register r is
  // kb0 + 8 (r/4) + 4 hh + r%4).  The range test runs only in tiles flagged
  // dirty (at most three per row of tiles), which keeps it off the scalar
  // unit in every other tile.
  auto mask = [&](f32x16& s, int kb0, unsigned mword, bool dirty) ULYS_INLINE {
    if ((dirty && straddles(kb0)) || (MASK && mword != ~0u)) {
      const unsigned vbits = __builtin_amdgcn_readfirstlane(valid_bits(kb0, mword));
      // (volatile: keeps this lane-dependent work inside the rarely taken branch)
      unsigned lb;
      asm volatile("v_lshrrev_b32 %0, %1, %2" : "=v"(lb) : "v"(4 * hh), "s"(vbits));
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = ((lb >> (8 * (r >> 2) + (r & 3))) & 1u) ? s[r] : -INFINITY;
    }
  };

  // This lane's max over its 16 scores of a block (raw scores).
  auto part_max = [&](const f32x16& s) ULYS_INLINE {
    float m = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, s[r]), s[r + 1]);
    return fmaxf(m, s[15]);
  };

  // Probabilities exp2(c log2e s - m_run) of accumulator registers 8e..8e+7
  // -> bf16 B operand p[e] of the PV MFMA, and their fp32 sums in two chains.
  auto probs_pair = [&](const f32x16& s, int e, int i, bf16x8 (&p)[2], float& ls0, float& ls1, int rh) ULYS_INLINE {
    const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * e + 2 * i], c2, negm[rh]));
    const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * e + 2 * i + 1], c2, negm[rh]));
    const f32x2 xx = {x0, x1};
    const bf16x2 pk = __builtin_convertvector(xx, bf16x2);
    p[e][2 * i] = pk[0];
    p[e][2 * i + 1] = pk[1];
    if (e == 0 && i == 0) { ls0 = x0; ls1 = x1; } else { ls0 += x0; ls1 += x1; }
  };
  auto probs = [&](const f32x16& s, bf16x8 (&p)[2], float& ls0, float& ls1, int rh) ULYS_INLINE {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) probs_pair(s, e, i, p, ls0, ls1, rh);
  };

  // The probabilities and sums are complete here (the empty asm consumes
  // them), so the compiler keeps their VALU work among the MFMAs issued before
  // this point instead of sinking it past the rescale branch.
  auto pin = [&](const bf16x8 (&pp)[2], float ls0, float ls1) ULYS_INLINE {
    asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pp[0])), "v"(__builtin_bit_cast(u32x4, pp[1])), "v"(ls0),
                 "v"(ls1));
  };

  // Raising the running max (rare: a few times per row).  The PV MFMAs of the
  // previous block were formed with the old max and are already accumulated,
  // so O and l are rescaled by exp2(m_old - m_new); this block's scores are
  // recomputed from K in LDS, their max taken, and the probabilities redone
  // with the new max.
  auto raise_max = [&](int kdelta, int kb, int kb0, unsigned mword, bool dirty, bf16x8 (&p)[2], float& ls0,
                       float& ls1, int rh) ULYS_INLINE {
    KFrag kf;
    read_k(kdelta, kb, kf);
    f32x16 s = qk(kf, rh);
    mask(s, kb0, mword, dirty);
    const float mx = lane_swap_max(part_max(s)) * c2;
    const float mn = fmaxf(m_run[rh], mx);
    const float alpha = (mn == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run[rh] - mn);
    m_run[rh] = mn;
    negm[rh] = (mn == -INFINITY) ? 0.0f : -mn;
    thr[rh] = (mn == -INFINITY) ? -1.0f : kLazySum;
    l_run[rh] *= alpha;
    settle_o(rh);
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[rh][db][r] *= alpha;
    settle_o_written(rh);
    probs(s, p, ls0, ls1, rh);
    // (two row halves: the new probabilities settle before an asm PV MFMA reads them)
    if constexpr (NH == 2) asm volatile("s_nop 1" : "+v"(p[0]), "+v"(p[1]));
  };

  // ---- software pipeline over 32-key blocks ----
  // Iteration b holds S(b) (scores), the V^T operands of block b-1 and its
  // probabilities P(b-1).  It issues the K reads of block b+1, forms P(b)
  // speculatively with the current max (VALU), accumulates PV(b-1) and computes
  // S(b+1) (MFMA, independent of the softmax of b), reads V(b), and only then
  // checks whether block b raises the max.  The LDS ring has three stages: a
  // tile is read from the iteration before its first block to its last block.
  // Scores and probabilities alternate between two register sets from one
  // block to the next (S(b) in one, S(b+1) in the other), so no copies.
  f32x16 sA[NH], sB[NH];
  VFrag vf;
  bf16x8 pA[NH][2], pB[NH][2];

  constexpr int kPVMfma = 2 * C::kDB;
  constexpr int kQKMfma = C::kQKSteps;

  // Block b: s_in = S(b), p_in = P(b-1), vf = V(b-1) operands.  Produces
  // s_out = S(b+1) (K of stage st_next, block kb_next), p_out = P(b), and
  // vf = V(b) operands (stage st, block kb).  kb0 = first key of block b,
  // mword = its key-mask word.  read_next(i, kf, part): part 0 reads K
  // operand i of block b+1 into kf; part 1 is side work for the caller (only
  // called with two row halves).
  auto iteration = [&](auto read_next, auto st, int kdelta, auto kb, int kb0, unsigned mword, bool dirty,
                       f32x16 (&s_in)[NH], f32x16 (&s_out)[NH], bf16x8 (&p_in)[NH][2],
                       bf16x8 (&p_out)[NH][2]) ULYS_INLINE {
    // (two row halves: a dirty block masks its scores right away, so it first
    // waits out the 12 wait states after the QK^T MFMAs that wrote them)
    if constexpr (NH == 2) {
      if (dirty) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(s_in[0]), "+v"(s_in[1]));
    }
#pragma unroll
    for (int rh = 0; rh < NH; ++rh) mask(s_in[rh], kb0, mword, dirty);
    KFrag kf;
    float ls0[NH], ls1[NH];
    f32x16 sn[NH];
    if constexpr (NH == 2) {
      // One wave per SIMD, so nothing else covers its stalls: both phases are
      // placed by hand at one MFMA per issue group (the scheduler may not move
      // work across a group boundary).  Beside each MFMA sits one step of the
      // probability pipeline and at most one LDS read or tile load.
      //
      // The block's 32 probability elements per lane (element m: row half
      // m % 2, score m / 2 of the PV phase's half of the keys, then of the QK^T
      // phase's half) run through three stages, one group apart: scaled score
      // (fma), exponential, then row sum and bf16 pack.  Stage r does the
      // first of element r, the second of r-1 and the third of r-2; the 34
      // stages are spread over the 32 groups (two in groups 14 and 29) so that
      // the pipeline drains before the last MFMA instead of after it.  Each
      // lane's two row sums add their elements in the same order as the
      // two-wave shape, so the sums are bit-identical.
      float tt[32], xx[32];
      auto e_h = [](int m) { return m & 1; };
      auto e_idx = [](int m) { return m < 16 ? (m >> 1) : 8 + ((m - 16) >> 1); };
      auto stage = [&](int r) ULYS_INLINE {
        if (r < 32) tt[r] = __builtin_fmaf(s_in[e_h(r)][e_idx(r)], c2, negm[e_h(r)]);
        if (r >= 1 && r - 1 < 32) xx[r - 1] = __builtin_amdgcn_exp2f(tt[r - 1]);
        if (r >= 2 && r - 2 < 32) {
          const int m = r - 2, h = e_h(m), idx = e_idx(m);
          const float x = xx[m];
          if ((idx & 1) == 0) {
            if (idx == 0) ls0[h] = x; else ls0[h] += x;
          } else {
            if (idx == 1) ls1[h] = x; else ls1[h] += x;
            const f32x2 v2 = {xx[m - 2], x};
            const bf16x2 pk = __builtin_convertvector(v2, bf16x2);
            p_out[h][idx >> 3][(idx & 7) - 1] = pk[0];
            p_out[h][idx >> 3][idx & 7] = pk[1];
          }
        }
      };
      // PV phase: group (g, rh) accumulates O[rh] over V fragment g; beside it
      // the K read g of block b+1 (rh = 0) or the caller's side work (rh = 1,
      // a clean step's tile load).
#pragma unroll
      for (int g = 0; g < kPVMfma; ++g) {
        const int db = g % C::kDB, e = g / C::kDB;
#pragma unroll
        for (int rh = 0; rh < NH; ++rh) {
          pv_one(o[rh][db], vf.x[db][e], p_in[rh][e]);
          const int r = 2 * g + rh;   // 0..15
          if (r < 14) stage(r); else if (r == 14) { stage(14); stage(15); } else stage(16);
          read_next(g, kf, rh);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // QK^T phase: group (g, rh) is head-dim step g of S(b+1) for row half rh;
      // beside the first of each pair, the V read g of block b.
#pragma unroll
      for (int rh = 0; rh < NH; ++rh)
#pragma unroll
        for (int r = 0; r < 16; ++r) sn[rh][r] = 0.0f;
#pragma unroll
      for (int g = 0; g < kQKMfma; ++g) {
#pragma unroll
        for (int rh = 0; rh < NH; ++rh) {
          sn[rh] = qk_step(kf, g, sn[rh], rh);
          const int r = 16 + 2 * g + rh;   // 16..31
          if (r < 29) stage(r + 1); else if (r == 29) { stage(30); stage(31); } else stage(r + 2);
          if (rh == 0) read_v_one(v_of(st), kb, g % C::kDB, g / C::kDB, vf);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
    // phase 1: PV(b-1) MFMAs in explicit issue groups (the scheduler may not
    // move work across a group boundary), each V fragment feeding the MFMAs of
    // every row half, with a share of the K reads of block b+1 and of the first
    // half of the probabilities of block b beside them.
    // Wave priority: high outside the QK^T phase's body.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int g = 0; g < kPVMfma; ++g) {
      const int db = g % C::kDB, e = g / C::kDB;
#pragma unroll
      for (int rh = 0; rh < NH; ++rh) pv_one(o[rh][db], vf.x[db][e], p_in[rh][e]);
#pragma unroll
      for (int i = g * kKOffs / kPVMfma; i < (g + 1) * kKOffs / kPVMfma; ++i) read_next(i, kf, 0);
#pragma unroll
      for (int j = g * 4 * NH / kPVMfma; j < (g + 1) * 4 * NH / kPVMfma; ++j)
        probs_pair(s_in[j / 4], 0, j % 4, p_out[j / 4], ls0[j / 4], ls1[j / 4], j / 4);
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase 2: QK(b+1) MFMAs (each K fragment feeding every row half), the V
    // reads of block b and the second half of the probabilities, ordered by
    // the scheduler
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int rh = 0; rh < NH; ++rh)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[rh][r] = 0.0f;
#pragma unroll
    for (int g = 0; g < kQKMfma; ++g) {
#pragma unroll
      for (int rh = 0; rh < NH; ++rh) sn[rh] = qk_step(kf, g, sn[rh], rh);
#pragma unroll
      for (int j = g * (2 * C::kDB) / kQKMfma; j < (g + 1) * (2 * C::kDB) / kQKMfma; ++j)
        read_v_one(v_of(st), kb, j % C::kDB, j / C::kDB, vf);
#pragma unroll
      for (int j = g * 4 * NH / kQKMfma; j < (g + 1) * 4 * NH / kQKMfma; ++j)
        probs_pair(s_in[j / 4], 1, j % 4, p_out[j / 4], ls0[j / 4], ls1[j / 4], j / 4);
    }
    }
    // (two row halves: no wait states here.  S(b+1) is first read by VALU in
    // the next block's first probability step, which comes after this block's
    // max checks and the next block's first PV MFMA, more than 12 wait states
    // on; a dirty block, which masks its scores first, waits at its start)
    if constexpr (NH == 2) asm volatile("" : "+v"(sn[0]), "+v"(sn[1]));
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NH == 1) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int rh = 0; rh < NH; ++rh) {
      s_out[rh] = sn[rh];
      pin(p_out[rh], ls0[rh], ls1[rh]);
    }
#pragma unroll
    for (int rh = 0; rh < NH; ++rh) {
      const bool raise = __any(ls0[rh] + ls1[rh] > thr[rh]);
      if (NH == 2 ? __builtin_expect(raise, 0) : raise)   // (one wave per SIMD: the rare path out of line)
        raise_max(kdelta, kb, kb0, mword, dirty, p_out[rh], ls0[rh], ls1[rh], rh);
      l_run[rh] += ls0[rh] + ls1[rh];
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // Tiles in processing order: every tile with a valid key.  Without a key
  // mask these are all tiles except those wholly inside the gap; with one,
  // the workgroup lists them in LDS first (each thread tests a run of tiles,
  // then an exclusive scan of the counts places them).
  const int nskip = max(0, skip_last - skip_first);
  int nseq = ntiles - nskip;
  if constexpr (MASK) {
    const int per = (ntiles + kT - 1) / kT;
    const int t0 = min(tid * per, ntiles), t1 = min(t0 + per, ntiles);
    int cnt = 0;
    for (int t = t0; t < t1; ++t)   // (each thread its own tiles: lane-local bits)
      cnt += (valid_bits(t * kBN, mask_word(t * kBN)) | valid_bits(t * kBN + 32, mask_word(t * kBN + 32))) != 0u;
    int* scan = (int*)lds;   // the ring is not in use yet
    scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < kT; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    int pos = scan[tid] - cnt;
    nseq = scan[kT - 1];
    // (an entry's bit 15: every key of the tile valid; bit 14: the next tile is
    // listed too, so the two are consecutive in the sequence, and is not the
    // ragged last tile, whose rows past the end only the general step's
    // clamped loads may fetch -- a clean run loads one tile past its blocks)
    auto tile_valid = [&](int t) {
      return t < ntiles &&
             (valid_bits(t * kBN, mask_word(t * kBN)) | valid_bits(t * kBN + 32, mask_word(t * kBN + 32))) != 0u;
    };
    for (int t = t0; t < t1; ++t)
      if (tile_valid(t)) {
        const bool full = (valid_bits(t * kBN, mask_word(t * kBN)) & valid_bits(t * kBN + 32, mask_word(t * kBN + 32))) == ~0u;
        const bool link = t + 1 != tail_tile && tile_valid(t + 1);
        tile_list[pos++] = (unsigned short)(t | (full ? 0x8000 : 0) | (link ? 0x4000 : 0));
      }
    __syncthreads();
  }
  // Pieces of work: (query tile qtile, positions [p0, p0 + n) of the tile
  // sequence).  A key-range chunk is one piece: the split-th of `splits`
  // near-equal runs (a function of the tile sequence alone, the same for
  // every head).  A range of the sequence of units u = qtile * nunits + pos
  // is a run of pieces: the end of one tile, whole tiles, the start of
  // another.  (A mask that leaves no valid key gives each tile one empty
  // unit, so that its zero output is written.)
  // A range that starts inside a tile and runs past its end takes that
  // tile's tail last: every other piece starts at the first key tile, so the
  // workgroups of a launch keep walking the keys nearly in step (two key
  // positions, a fixed distance apart, at any time) and share K/V tiles in L2.
  const int nunits = max(nseq, 1);
  const long long units = (long long)a.qtiles * nunits;
  long long u = 0, uend = 1, ustart = 0, tail_u = -1, tail_end = -1;
  if (ranged) {
    ustart = u = (long long)wx * units / a.ranges;
    uend = (long long)(wx + 1) * units / a.ranges;
    const long long next_tile = (ustart / nunits + 1) * nunits;
    if (ustart % nunits != 0 && next_tile < uend) {
      tail_u = ustart;
      tail_end = next_tile;
      u = next_tile;
    }
  }
  if (ranged && wx == 0 && hl == 0 && tid == 0) a.range_nseq[b] = nseq;
  reset_kcur();
  for (;;) {
    if (u >= uend) {
      if (tail_u < 0) break;
      u = tail_u;
      uend = tail_end;
      tail_u = -1;
    }
    int qtile, p0, n;
    if (ranged) {
      qtile = (int)(u / nunits);
      p0 = (int)(u - (long long)qtile * nunits);
      n = (int)min(uend - u, (long long)(nunits - p0));
      if (nseq == 0) n = 0;
    } else {
      qtile = qtile0;
      p0 = (int)(((long long)split * nseq) / a.splits);
      n = (int)(((long long)(split + 1) * nseq) / a.splits) - p0;
    }
    const long long upiece = (long long)qtile * nunits + p0;
    u = ranged ? upiece + max(n, 1) : uend;
    const int qrow0 = qtile * kBM + wave * 32 * NH;
    load_q(qrow0);
    reset_state();
#pragma unroll
    for (int rh = 0; rh < NH; ++rh)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 8; ++i) pA[rh][e][i] = (__bf16)0.0f;
    // (two row halves: the zeros settle before the first asm PV MFMA reads them)
    if constexpr (NH == 2) asm volatile("s_nop 1" : "+v"(pA[0][0]), "+v"(pA[0][1]), "+v"(pA[1][0]), "+v"(pA[1][1]));

    // (uniform across the workgroup: kept in scalar registers)
    auto seq_tile = [&](int pos) {
      pos += p0;
      if constexpr (MASK) return __builtin_amdgcn_readfirstlane((int)(tile_list[pos] & 0x0FFF));
      else return pos < skip_first ? pos : pos + nskip;
    };
    // Position pos goes to stage pos % kStages; past the end the last tile is
    // loaded again, which keeps every wave's load count per tile uniform.
    auto load_pos = [&](int pos, auto st) { load_tile(seq_tile(min(pos, n - 1)), st); };

    if (n > 0) {   // else (an empty chunk, or a mask that left no valid key) o = 0, lse = -inf
      load_pos(0, std::integral_constant<int, 0>{});
      load_pos(1, std::integral_constant<int, 1>{});
      if constexpr (kStages > 3) load_pos(2, std::integral_constant<int, 2>{});
      __builtin_amdgcn_s_waitcnt(0x0070);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      {
        KFrag kf;
        read_k(-C::kKTile, B0{}, kf);
#pragma unroll
        for (int rh = 0; rh < NH; ++rh) sA[rh] = qk(kf, rh);
        read_v(v_of(B0{}), B0{}, vf);   // finite operands for the empty PV of block -1
      }
      int tc = seq_tile(0);
      // Visited tiles with keys outside [0, rows) or inside the gap ("dirty":
      // their blocks take the per-block range test): the one holding the gap's
      // first key, the one holding its last, and the ragged last tile.  Each
      // visited tile is compared with all three (the gap's last tile may be
      // wholly inside the gap and never visited, so no running "next dirty
      // tile" can be kept).
      constexpr int kNone = 0x7fffffff;
      const int dz = tail_tile >= 0 ? tail_tile : kNone;
      const int dx = gs < ge ? gs / kBN : dz, dy = gs < ge ? (ge - 1) / kBN : dz;
      auto is_dirty = [&](int t) { return t == dx || t == dy || t == dz; };
      bool dc = is_dirty(tc);
      // mask words of the tile's second block (mw1) and of the next tile's blocks
      // (fetched a block ahead: each is a scalar value once it is used)
      unsigned mw1 = mask_word(tc * kBN + 32);
      iteration([&](int i, KFrag& kf, int part) ULYS_INLINE { if (part == 0) read_k_one(-C::kKTile, B1{}, i, kf); }, B0{}, -C::kKTile, B0{},
                tc * kBN,
                __builtin_amdgcn_readfirstlane(mask_word(tc * kBN)), dc, sA, sB, pA, pB);
      tile_barrier();

      // Position i (stage SA): its second block, then the first block of
      // position i+1 (stage SB).  Position i + kStages - 1 is loaded first, into
      // SP, the stage of position i-1, which every wave has finished with.  The
      // next tile's key-mask words are fetched a block ahead.  Each step ends
      // with a barrier.  Returns false after the last position.
      auto step = [&](int i, auto SA, auto SB, auto SP) ULYS_INLINE {
        load_pos(i + kStages - 1, SP);
        const int tn = i + 1 < n ? seq_tile(i + 1) : tc;
        const unsigned wn0 = mask_word(tn * kBN), wn1 = mask_word(tn * kBN + 32);
        iteration([&](int i, KFrag& kf, int part) ULYS_INLINE { if (part == 0) read_k_one(0, B0{}, i, kf); }, SA, (int(SA) - int(SB)) * C::kKTile, B1{},
                  tc * kBN + 32,
                  __builtin_amdgcn_readfirstlane(mw1), dc, sB, sA, pB, pA);
        if (i + 1 >= n) return false;
        tc = tn;
        mw1 = wn1;
        dc = is_dirty(tc);
        iteration([&](int i, KFrag& kf, int part) ULYS_INLINE { if (part == 0) read_k_one(0, B1{}, i, kf); }, SB, 0, B0{}, tc * kBN,
                  __builtin_amdgcn_readfirstlane(wn0), dc, sA, sB, pA, pB);
        // the next step reads K from the stage after SB
        const int adv = int(SB) == kStages - 1 ? -(kStages - 1) * C::kKTile : C::kKTile;
#pragma unroll
        for (int k = 0; k < kKOffs; ++k) kcur[k] += adv;
        tile_barrier();
        return true;
      };
      int sa = 0;
      // Clean steps: while every tile a step touches (positions i and i+1, and
      // the load of i+2) is clean and on one side of the gap, consecutive
      // positions hold consecutive tiles, so a step needs no dirty tests and
      // its tile load is the previous one's plus one tile (two pointer
      // increments instead of the tile-index arithmetic).  The steps of a
      // clean run take the K read offsets at stage 0, so a read of stage s is
      // the offset plus s * kKTile; in whole ring rounds the stages are
      // compile-time constants, and every LDS read and tile-load address is a
      // register plus an immediate with no address arithmetic at all
      // (measured +2-3% at two and ten heads, +7% at one).
      const unsigned char* ktp = kbase;
      const unsigned char* vtp = vbase;
      auto clean_step = [&](auto SA, auto SB, auto SP) ULYS_INLINE {
        const unsigned int kl = lds_u32(k_of(SP)) + kls;
        const unsigned int vl = lds_u32(v_of(SP) + kVRegion) + vls;
        const int ka = int(SA) * C::kKTile, kbb = int(SB) * C::kKTile;
        // With one wave per SIMD a burst of tile loads would stall the wave's
        // MFMAs: its eight loads go one each beside the second row half's PV
        // MFMAs of the step's first block instead.
        constexpr bool kSpread = NH == 2;
        static_assert(!kSpread || kKSegsPerWave + kVSegsPerWave == kKOffs, "one tile load per PV group");
        if constexpr (kSpread) {
          iteration([&](int i, KFrag& kf, int part) ULYS_INLINE {
                      if (part == 0) { read_k_one(kbb, B0{}, i, kf); return; }
                      if (i < kKSegsPerWave) dma16(ktp, kgo_u[i], kl + i * kW * 1024);
                      else dma16(vtp, vgo_u[i - kKSegsPerWave], vl + (i - kKSegsPerWave) * kW * 1024);
                    }, SA, ka, B1{}, 0, ~0u, false, sB, sA, pB, pA);
          ktp += ktile;
          vtp += vtile;
        } else {
#pragma unroll
          for (int u = 0; u < kKSegsPerWave; ++u) dma16(ktp, kgo_u[u], kl + u * kW * 1024);
#pragma unroll
          for (int u = 0; u < kVSegsPerWave; ++u) dma16(vtp, vgo_u[u], vl + u * kW * 1024);
          ktp += ktile;
          vtp += vtile;
          iteration([&](int i, KFrag& kf, int part) ULYS_INLINE { if (part == 0) read_k_one(kbb, B0{}, i, kf); },
                    SA, ka, B1{}, 0, ~0u, false, sB, sA, pB, pA);
        }
        iteration([&](int i, KFrag& kf, int part) ULYS_INLINE { if (part == 0) read_k_one(kbb, B1{}, i, kf); },
                  SB, kbb, B0{}, 0, ~0u, false, sA, sB, pA, pB);
        tile_barrier();
      };
      // Clean steps from step i.  Without a key mask the first tile at or after
      // step i's that is dirty, or the side of the gap ending, ends the run;
      // with one the run lasts while the listed tiles are full (every key
      // valid) and consecutive, so their blocks need no mask either.
      auto clean_run = [&](int i) -> int {
        if constexpr (MASK) {
          // positions from p0 + i whose tile is full and followed by the next
          // tile, found 64 at a time by a wave ballot (the same in every wave)
          const int room = n - 2 - i;
          if (room <= 0) return 0;
          const int q = p0 + i;
          int k = 0;
          for (;;) {
            const int p = q + k + (fresh_tid() & 63);
            const bool ok = p < nseq && (tile_list[p] & 0xC000) == 0xC000;
            const unsigned long long bad = __ballot(!ok);
            if (bad != 0ull) { k += __builtin_ctzll(bad); break; }
            k += 64;
            if (k > room) break;
          }
          return __builtin_amdgcn_readfirstlane(max(0, min(room, k - 1)));
        }
        const int room = n - 2 - i;   // steps whose tile load stays inside the piece
        const int q = p0 + i;
        int t0, tend;
        if (q + 2 < skip_first) { t0 = q; tend = skip_first; }        // before the gap
        else if (q >= skip_first) { t0 = q + nskip; tend = ntiles; }   // after it
        else return 0;                                                   // the step crosses it
        const int d = dx >= t0 ? dx : dy >= t0 ? dy : dz >= t0 ? dz : kNone;   // (dx <= dy <= dz)
        return max(0, min(room, min(tend, d) - t0 - 2));
      };
      // Whole ring rounds of clean steps from step i (the ring at stage 0,
      // so sa = 0 and the K offsets point at stage 1); the steps short of a
      // round take the general step.
      auto run_clean = [&](int i, int rounds) {
        static_assert(kStages == 3, "a clean round is three steps, one per stage");
        using S0 = std::integral_constant<int, 0>;
        using S1 = std::integral_constant<int, 1>;
        using S2 = std::integral_constant<int, 2>;
        ktp = kbase + (size_t)(unsigned int)seq_tile(i + 2) * ktile;
        vtp = vbase + (size_t)(unsigned int)seq_tile(i + 2) * vtile;
#pragma unroll
        for (int k = 0; k < kKOffs; ++k) kcur[k] -= C::kKTile;
        for (int r = 0; r < rounds; ++r) {
          clean_step(S0{}, S1{}, S2{});
          clean_step(S1{}, S2{}, S0{});
          clean_step(S2{}, S0{}, S1{});
        }
#pragma unroll
        for (int k = 0; k < kKOffs; ++k) kcur[k] += C::kKTile;
        tc = seq_tile(i + rounds * kStages);
        dc = is_dirty(tc);
        if constexpr (MASK) mw1 = mask_word(tc * kBN + 32);
      };
      for (int i = 0;; ++i) {
        if (sa == 0) {
          const int rounds = clean_run(i) / kStages;
          if (rounds > 0) {
            run_clean(i, rounds);
            i += rounds * kStages;
          }
        }
        const int sb = sa == kStages - 1 ? 0 : sa + 1;
        if (!step(i, sa, sb, sa == 0 ? kStages - 1 : sa - 1)) break;
        sa = sb;
      }
      pv(vf, pA);
      // back to the first step's K offsets (the last step, at stage sa, read
      // K from stage sa + 1 and did not move them)
      const int kback = ((sa == kStages - 1 ? 0 : sa + 1) - 1) * C::kKTile;
#pragma unroll
      for (int k = 0; k < kKOffs; ++k) kcur[k] -= kback;
    }

    // ---- epilogue: normalise, write o (bf16) and lse (fp32, natural log) ----
    // (a key-range chunk, or a range's piece of a tile it shares with other
    // ranges: o in fp32 and lse in the log2 domain, to be merged)
    // The rows leave through this wave's LDS staging area, 128 bytes of each
    // row at a time: a global store then covers whole 128-byte lines (8 lanes
    // per line) instead of 16 bytes of 32 different rows.
    const int ft = fresh_tid();
    const int l32f = ft & 31, hhf = (ft >> 5) & 1, lanef = ft & 63;
    // (written directly: a whole tile; else fp32 partials to be merged)
    const bool whole = ranged ? (p0 == 0 && n == nseq) : a.splits <= 1;
    constexpr int kRW = 32 * NH;   // rows of this wave
    unsigned char* const stg = stage_lds + wave * kRW * kStgPitch;
    float inv[NH], lse2[NH];
#pragma unroll
    for (int rh = 0; rh < NH; ++rh) {
      settle_o(rh);
      const float l = lane_swap_sum(l_run[rh]);
      inv[rh] = l > 0.0f ? 1.0f / l : 0.0f;
      lse2[rh] = l > 0.0f ? m_run[rh] + __log2f(l) : -INFINITY;
    }
    if (whole) {
#pragma unroll
      for (int c = 0; c < D / 64; ++c) {   // head dims [64c, 64c + 64): 128 bytes of bf16
#pragma unroll
        for (int rh = 0; rh < NH; ++rh)
#pragma unroll
          for (int dbi = 0; dbi < 2; ++dbi)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int db = 2 * c + dbi;
              const f32x2 lo = {o[rh][db][4 * r4 + 0] * inv[rh], o[rh][db][4 * r4 + 1] * inv[rh]};
              const f32x2 hi = {o[rh][db][4 * r4 + 2] * inv[rh], o[rh][db][4 * r4 + 3] * inv[rh]};
              u32x2 w;
              w.x = __builtin_bit_cast(unsigned int, __builtin_convertvector(lo, bf16x2));
              w.y = __builtin_bit_cast(unsigned int, __builtin_convertvector(hi, bf16x2));
              *(u32x2*)(stg + (rh * 32 + l32f) * kStgPitch + (dbi * 32 + 8 * r4 + 4 * hhf) * 2) = w;
            }
#pragma unroll
        for (int kq = 0; kq < kRW / 8; ++kq) {
          const int lr = kq * 8 + (lanef >> 3), ch = lanef & 7;
          const u32x4 x = *(const u32x4*)(stg + lr * kStgPitch + ch * 16);
          const int row = qrow0 + lr;
          if (row < qrows)
            *(u32x4*)(a.o + ((size_t)b * qrows + row) * q_row_stride + (size_t)head * D + c * 64 + ch * 8) = x;
        }
      }
#pragma unroll
      for (int rh = 0; rh < NH; ++rh) {
        const int row = qrow0 + rh * 32 + l32f;
        if (a.lse != nullptr && hhf == 0 && row < qrows)
          a.lse[((size_t)b * a.hq + head) * qrows + row] = lse2[rh] * kLn2;
      }
    } else {
      // fp32 rows: a key-range chunk's at its (split, b, row, head) position, a
      // cut tile's piece in slot 0 (the range's first piece) or 1 (its last)
      const bool keysplit = !ranged;
      const size_t pidx = (((size_t)b * a.hsub + hl) * a.ranges + wx) * 2 + (upiece == ustart ? 0 : 1);
      auto prow = [&](int row) -> float* {
        if (keysplit) return a.part_o + ((((size_t)split * a.batch + b) * qrows + row) * a.hsub + hl) * D;
        return a.part_o + (pidx * kBM + (row - qtile * kBM)) * D;
      };
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {   // head dims [32c, 32c + 32): 128 bytes of fp32
#pragma unroll
        for (int rh = 0; rh < NH; ++rh)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 w = {o[rh][c][4 * r4 + 0] * inv[rh], o[rh][c][4 * r4 + 1] * inv[rh],
                              o[rh][c][4 * r4 + 2] * inv[rh], o[rh][c][4 * r4 + 3] * inv[rh]};
            *(f32x4*)(stg + (rh * 32 + l32f) * kStgPitch + (8 * r4 + 4 * hhf) * 4) = w;
          }
#pragma unroll
        for (int kq = 0; kq < kRW / 8; ++kq) {
          const int lr = kq * 8 + (lanef >> 3), ch = lanef & 7;
          const f32x4 x = *(const f32x4*)(stg + lr * kStgPitch + ch * 16);
          const int row = qrow0 + lr;
          if (row < qrows) *(f32x4*)(prow(row) + c * 32 + ch * 4) = x;
        }
      }
#pragma unroll
      for (int rh = 0; rh < NH; ++rh) {
        const int row = qrow0 + rh * 32 + l32f;
        if (hhf == 0 && row < qrows) {
          if (keysplit) a.part_lse[(((size_t)split * a.batch + b) * a.hsub + hl) * qrows + row] = lse2[rh];
          else a.part_lse[pidx * kBM + (row - qtile * kBM)] = lse2[rh];
        }
      }
    }
    if (u < uend || tail_u >= 0) {
      // the next piece refills the ring: every tile load of this one has
      // landed and every wave is done reading it
      __builtin_amdgcn_s_waitcnt(0x0070);
      asm volatile("" ::: "memory");
      __syncthreads();
    }
  }
}

// Merge of the key-range splits of one launch, in split order (fixed, so the
// result does not depend on which workgroup finished first):
//   M = max_s lse_s,  w_s = 2^(lse_s - M),  o = sum_s w_s o_s / sum_s w_s,
//   lse = (M + log2 sum_s w_s) ln 2,
// the exact combination of softmaxes over disjoint key sets (lse_s in the log2
// domain; a split with no key has lse_s = -inf and weight 0; if every split is
// empty, o = 0 and lse = -inf).  One thread per 8 head-dim elements of a
// (b, row, head): 2 x 16-byte fp32 reads per split, one 16-byte bf16 write.
constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void split_merge_kernel(AttnArgs a) {
  constexpr int kCpr = D / 8;   // threads per (b, row, head)
  const size_t total = (size_t)a.batch * a.q_rows * a.hsub * kCpr;
  const size_t idx = (size_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (idx >= total) return;
  const int c = (int)(idx % kCpr);
  const size_t rh = idx / kCpr;               // (b * q_rows + row) * hsub + hl
  const int hl = (int)(rh % a.hsub);
  const size_t br = rh / a.hsub;              // b * q_rows + row
  const int row = (int)(br % a.q_rows);
  const int b = (int)(br / a.q_rows);
  const size_t split_o = (size_t)a.batch * a.q_rows * a.hsub * D;       // floats per split
  const size_t split_l = (size_t)a.batch * a.hsub * a.q_rows;
  const size_t li = ((size_t)b * a.hsub + hl) * a.q_rows + row;

  float lv[kMaxKeySplits];
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxKeySplits; ++s)
    if (s < a.splits) {
      lv[s] = a.part_lse[s * split_l + li];
      mx = fmaxf(mx, lv[s]);
    }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.0f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int s = 0; s < kMaxKeySplits; ++s)
      if (s < a.splits) {
        const float w = __builtin_amdgcn_exp2f(lv[s] - mx);   // 0 for an empty split
        const f32x4* src = (const f32x4*)(a.part_o + s * split_o + rh * D + 8 * c);
        const f32x4 x0 = __builtin_nontemporal_load(src), x1 = __builtin_nontemporal_load(src + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] += w * x0[i];
          acc[4 + i] += w * x1[i];
        }
        wsum += w;
      }
  }
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 v = {acc[2 * i] * inv, acc[2 * i + 1] * inv};
    out[i] = __builtin_bit_cast(unsigned int, __builtin_convertvector(v, bf16x2));
  }
  const int head = a.head0 + hl;
  *(u32x4*)(a.o + (br * a.hq + head) * D + 8 * c) = out;
  if (a.lse != nullptr && c == 0)
    a.lse[((size_t)b * a.hq + head) * a.q_rows + row] = wsum > 0.0f ? (mx + __log2f(wsum)) * kLn2 : -INFINITY;
}

// Merge of a range split's cut tiles.  Workgroup: kBM / kMergeGroupsPerTile
// rows of one (query tile, head, b): several workgroups per tile, so that a
// CU holds several of them and their dependent load phases (the pieces' LSEs,
// then each piece's rows) overlap.  The tile's pieces come from the non-empty ranges between the one holding
// its first unit and the one holding its last (range of unit x: the largest
// r with r U / R <= x); a tile within one range was written by the attention
// kernel and is skipped.  Combination in range order, as for key-range
// chunks: M = max lse_r, w_r = 2^(lse_r - M), o = sum_r w_r o_r / sum_r w_r,
// lse = (M + log2 sum_r w_r) ln 2.  Thread: 4 head dims of kRowsPerPass rows
// (consecutive lanes read consecutive 16-byte chunks of a row), all of a
// piece's loads issued before they are used.
constexpr int kMergeGroupsPerTile = 4;

template <int D>
__global__ __launch_bounds__(kThreads) void range_merge_kernel(AttnArgs a) {
  constexpr int kC4 = D / 4;                     // 16-byte chunks per row
  constexpr int kRowsPerPass = kThreads / kC4;   // rows the workgroup covers at once
  constexpr int kRowsPerGroup = kBM / kMergeGroupsPerTile;
  constexpr int kPasses = kRowsPerGroup / kRowsPerPass;
  static_assert(kPasses >= 1 && kRowsPerGroup % kRowsPerPass == 0, "whole passes per workgroup");
  const int qtile = blockIdx.x / kMergeGroupsPerTile, hl = blockIdx.y, b = blockIdx.z;
  const int rbase = (blockIdx.x % kMergeGroupsPerTile) * kRowsPerGroup;   // this workgroup's rows of the tile
  const long long nunits = max(a.range_nseq[b], 1);
  const long long units = (long long)a.qtiles * nunits, R = a.ranges;
  auto range_start = [&](long long r) { return r * units / R; };
  auto range_of = [&](long long x) { return (int)(((x + 1) * R - 1) / units); };
  const long long t0 = (long long)qtile * nunits;
  const int rf = range_of(t0), rl = range_of(t0 + nunits - 1);
  if (rf == rl) return;   // (a range holds the whole tile)
  const int c4 = threadIdx.x % kC4, r0 = rbase + threadIdx.x / kC4;
  const size_t pbase = ((size_t)b * a.hsub + hl) * (size_t)R;
  auto piece = [&](int r) { return ((pbase + r) * 2 + (range_start(r) < t0 ? 1 : 0)) * kBM; };
  auto nonempty = [&](int r) { return range_start(r + 1) > range_start(r); };
  float mx[kPasses], wsum[kPasses];
  f32x4 acc[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    mx[p] = -INFINITY;
    wsum[p] = 0.0f;
    acc[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int r = rf; r <= rl; ++r)
    if (nonempty(r)) {
      const size_t pi = piece(r);
#pragma unroll
      for (int p = 0; p < kPasses; ++p) mx[p] = fmaxf(mx[p], a.part_lse[pi + p * kRowsPerPass + r0]);
    }
  for (int r = rf; r <= rl; ++r)
    if (nonempty(r)) {
      const size_t pi = piece(r);
      float lv[kPasses];
      f32x4 x[kPasses];
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
        const size_t row = pi + p * kRowsPerPass + r0;
        lv[p] = a.part_lse[row];
        x[p] = __builtin_nontemporal_load((const f32x4*)(a.part_o + row * D) + c4);
      }
#pragma unroll
      for (int p = 0; p < kPasses; ++p)
        if (mx[p] != -INFINITY) {
          const float w = __builtin_amdgcn_exp2f(lv[p] - mx[p]);   // 0 for a piece with no key
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[p][j] += w * x[p][j];
          wsum[p] += w;
        }
    }
  const int head = a.head0 + hl;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    const int row = qtile * kBM + p * kRowsPerPass + r0;
    if (row >= a.q_rows) continue;
    const float inv = wsum[p] > 0.0f ? 1.0f / wsum[p] : 0.0f;
    const f32x2 lo = {acc[p][0] * inv, acc[p][1] * inv}, hi = {acc[p][2] * inv, acc[p][3] * inv};
    u32x2 out;
    out.x = __builtin_bit_cast(unsigned int, __builtin_convertvector(lo, bf16x2));
    out.y = __builtin_bit_cast(unsigned int, __builtin_convertvector(hi, bf16x2));
    *(u32x2*)(a.o + (((size_t)b * a.q_rows + row) * a.hq + head) * D + 4 * c4) = out;
    if (a.lse != nullptr && c4 == 0)
      a.lse[((size_t)b * a.hq + head) * a.q_rows + row] = wsum[p] > 0.0f ? (mx[p] + __log2f(wsum[p])) * kLn2 : -INFINITY;
  }
}

template <int D, bool FP8>
hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.ranges > 0 ? a.ranges : a.qtiles * a.splits, a.hsub, a.batch);
  constexpr int kNHm = kRowHalves<D, FP8, true>, kNH = kRowHalves<D, FP8, false>;
  if (a.key_mask != nullptr)
    hipLaunchKernelGGL((attn_fwd_kernel<D, FP8, true, kNHm>), grid, dim3(kThreads / kNHm), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, FP8, false, kNH>), grid, dim3(kThreads / kNH), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ranges > 0) {
    hipLaunchKernelGGL((range_merge_kernel<D>), dim3(a.qtiles * kMergeGroupsPerTile, a.hsub, a.batch),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  if (a.splits == 1) return hipSuccess;
  const size_t threads = (size_t)a.batch * a.q_rows * a.hsub * (D / 8);
  hipLaunchKernelGGL((split_merge_kernel<D>), dim3((unsigned)((threads + kMergeThreads - 1) / kMergeThreads)),
                     dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

// Workspace of a split launch: fp32 partial o and lse per head (key-range
// split: every chunk of every row; range split: two tile pieces per range),
// then one int per batch (the range split's tile count).
WorkspaceSize workspace_size(const AttnArgs& a, int D) {
  WorkspaceSize w{0, 0, 0, 0};
  if (a.ranges > 0) {
    w.o_per_head = (size_t)a.batch * a.ranges * 2 * kBM * D * sizeof(float);
    w.lse_per_head = (size_t)a.batch * a.ranges * 2 * kBM * sizeof(float);
  } else if (a.splits > 1) {
    w.o_per_head = (size_t)a.splits * a.batch * a.q_rows * D * sizeof(float);
    w.lse_per_head = (size_t)a.splits * a.batch * a.q_rows * sizeof(float);
  } else {
    return w;
  }
  w.fixed = ((size_t)a.batch * sizeof(int) + 255) & ~(size_t)255;
  w.per_head = w.o_per_head + w.lse_per_head;
  return w;
}

template <int D, bool FP8>
hipError_t launch(const AttnArgs& in, void* ws, size_t ws_bytes, hipStream_t s) {
  AttnArgs a = in;
  a.qtiles = (a.q_rows + kBM - 1) / kBM;
  a.head0 = 0;
  a.hsub = a.hq;
  if (a.ranges > 0) a.splits = 1;
  if (a.splits <= 1 && a.ranges == 0) {
    a.splits = 1;
    return launch_one<D, FP8>(a, s);
  }
  // The caller's workspace holds the partials of hsub heads at a time (the
  // host checked that it holds at least one head's); a call over more heads
  // runs as several launches over head ranges (each head's bytes unchanged).
  const WorkspaceSize w = workspace_size(a, D);
  const int hsub = (int)std::min<size_t>((size_t)a.hq, (ws_bytes - w.fixed) / w.per_head);
  a.range_nseq = (int*)ws;
  a.part_o = (float*)((char*)ws + w.fixed);
  a.part_lse = (float*)((char*)a.part_o + w.o_per_head * hsub);
  for (int h0 = 0; h0 < a.hq; h0 += hsub) {
    a.head0 = h0;
    a.hsub = std::min(hsub, a.hq - h0);
    const hipError_t e = launch_one<D, FP8>(a, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

WorkspaceSize attn_workspace_size(const AttnArgs& a, int head_dim) { return workspace_size(a, head_dim); }

hipError_t launch_attn(const AttnArgs& a, int head_dim, bool fp8, void* ws, size_t ws_bytes, hipStream_t s) {
  if (head_dim == 128) return fp8 ? launch<128, true>(a, ws, ws_bytes, s) : launch<128, false>(a, ws, ws_bytes, s);
  return fp8 ? launch<64, true>(a, ws, ws_bytes, s) : launch<64, false>(a, ws, ws_bytes, s);
}

// ---- static scratch for callers that cannot allocate ----
// The workspace of ulys_attend_group_noalloc: one array per GPU, alive until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// the device array: kernels get the device address that hipGetSymbolAddress
// returns for the current device, looked up once per device and cached.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];
}  // namespace

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kScratchDevices;
  if (cached) {
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p != nullptr) {
      *out = p;
      return hipSuccess;
    }
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  if (cached) g_scratch[dev].store(p, std::memory_order_release);   // every thread finds the same address
  *out = p;
  return hipSuccess;
}

}  // namespace ulys
