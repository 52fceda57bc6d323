// Internal declarations shared by the libulys translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ulys {

constexpr int kMaxDegree = 64;      // P shards per call (kernel-argument arrays)
constexpr int kMaxGapBatch = 256;   // batches that may carry a key gap
constexpr int kMaxPipelineGroups = 64;   // head groups of one ulys_rank_pipeline call
constexpr int kMaxMergeParts = 16;       // partial results of one ulys_lse_merge call
constexpr int kAttnRowsPerWorkgroup = 256;   // query rows per attention workgroup (one per CU at a time)
constexpr int kAttnKeysPerTile = 64;         // keys per attention LDS tile
constexpr int kMaxMaskTiles = 4096;          // key tiles (262144 keys) an attention call with a key mask may span
constexpr int kMaxKeySplits = 16;            // key-range chunks per query tile
constexpr int kMaxRanges = 4096;             // ranges per (batch, head) of a range split
constexpr int kMaxRangesPerTile = 32;        // ... and per query tile
constexpr int kMaxAmaxTensors = 64;

// Geometry of one pack/unpack launch, resolved on the host.
struct RepackGeom {
  int batch, rows, s_local, n_rep, rep_first, rank, degree, shard_rows, head_dim;
  int ngroups;   // groups handled by this launch (1, or all G)
};

struct PackArgs {
  RepackGeom g[3];                     // q, k, v (a K/V-only prefix gives q its own geometry)
  const uint16_t* src[3][kMaxDegree];  // q, k, v shards
  void* dst[3];                        // q, k, v slots
  int heads[3];                        // heads of the source tensor (Hq, Hkv, Hkv)
  int gh[3];                           // heads per group
  int h0[3];                           // first head of the first group of this launch
  int fp8[3];                          // 1: cast to e4m3fn (q, k only)
  const float* amax;                   // device {amax_q, amax_k} when fp8
};

struct UnpackArgs {
  RepackGeom g;
  const uint16_t* src;                 // o slot(s)
  uint16_t* dst[kMaxDegree];           // o shards
  int heads, gh, h0;
};

struct AmaxArgs {
  const uint16_t* src[kMaxAmaxTensors];
  int n;
  size_t chunks_each;                  // 16-byte chunks per tensor
  unsigned int* out;                   // float bits of max |x|
};

struct MergeArgs {
  const uint16_t* o[kMaxMergeParts];   // partial outputs [B, rows, heads, D] bf16
  const float* lse[kMaxMergeParts];    // partial LSEs [B, heads, rows]
  int n;
  uint16_t* out;                       // merged output
  float* lse_out;                      // merged LSE or null
  int batch, rows, heads, head_dim;
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  uint16_t* o;
  float* lse;
  const float* amax;                   // fp8 q/k: device {amax_q, amax_k}
  float scale;                         // softmax scale (before fp8 descale)
  int batch, q_rows, kv_rows, hq, hkv;
  int has_gap;
  int gap[kMaxGapBatch][2];
  const uint32_t* key_mask;            // [batch][mask_words] valid-key bits, or null
  int mask_words;                      // ceil(kv_rows / 32)
  // Key-range split: `splits` workgroups share a (b, head, query tile), each
  // taking a contiguous run of its key tiles; with splits > 1 each writes its
  // fp32 result (o normalised, lse in the log2 domain) to part_o
  // [splits][batch][q_rows][hsub][D] / part_lse [splits][batch][hsub][q_rows]
  // and a merge kernel combines them in split order.  One launch covers heads
  // [head0, head0 + hsub).
  int splits, qtiles, head0, hsub;
  float* part_o;
  float* part_lse;
  // Range split (ranges = R > 0; splits is then 1): workgroup r of a
  // (b, head) takes units [r U / R, (r + 1) U / R) of the sequence
  // u = query tile * key tiles + key-tile position (U units), i.e. the end of
  // one query tile, whole tiles, the start of another.  A tile within one
  // range is written directly; the pieces of a tile cut by range ends leave
  // fp32 results in part_o [batch][hsub][R][2][kBM][D] / part_lse
  // [batch][hsub][R][2][kBM] (slot 0: the range's first piece, 1: its last)
  // for a merge kernel that combines them in range order.  range_nseq[b]:
  // key tiles with a valid key of batch b (written by the attention kernel).
  int ranges;
  int* range_nseq;
};

hipError_t launch_pack(const PackArgs& a, hipStream_t s);
hipError_t launch_unpack(const UnpackArgs& a, hipStream_t s);
hipError_t launch_amax(const AmaxArgs& a, hipStream_t s);
// Device workspace of a split attention launch (zero per_head: no split).
// A call needs fixed + per_head * heads bytes to run all heads in one launch,
// and at least fixed + per_head (one head per launch).
struct WorkspaceSize {
  size_t per_head;       // partial o + lse of one head
  size_t o_per_head;
  size_t lse_per_head;
  size_t fixed;          // the range split's per-batch tile counts (256-byte padded)
};
WorkspaceSize attn_workspace_size(const AttnArgs& a, int head_dim);   // a: splits/ranges resolved
hipError_t launch_attn(const AttnArgs& a, int head_dim, bool fp8, void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_lse_merge(const MergeArgs& a, hipStream_t s);

// Static scratch of ulys_attend_group_noalloc: kScratchBytes per GPU, held by
// the library from the first use on that GPU until the process ends.
constexpr size_t kScratchBytes = size_t(128) << 20;
// Device address of the current GPU's scratch (resolved once per device).
hipError_t scratch_address(void** out);

}  // namespace ulys
