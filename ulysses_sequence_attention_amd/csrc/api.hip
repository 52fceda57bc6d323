// libulys C ABI: argument validation and launch geometry (host side).
//
// Every rule is checked before anything touches the HIP runtime, so a bad
// call returns its status with nothing enqueued (and can be exercised on a
// machine without a GPU).  The library allocates nothing: device buffers,
// the attention workspace and the pipeline's events all belong to the
// caller.  The only state is the per-thread text of the last validation
// failure and a cache of each device's compute-unit count (atomic; a value
// the runtime reports the same way every time).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "../../include/ulys.h"
#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return ULYS_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Layout rules shared by pack and unpack.
int check_layout(const ulys_layout* L, int rank, int group) {
  if (L == nullptr) return fail(ULYS_EINVAL, "layout is NULL");
  if (L->batch < 1 || L->degree < 1 || L->s_local < 1 || L->hq < 1 || L->hkv < 1 || L->groups < 1)
    return fail(ULYS_EINVAL, "batch, degree, s_local, hq, hkv and groups must be >= 1");
  if (L->n_rep < 0) return fail(ULYS_EINVAL, "n_rep must be >= 0");
  if (L->rep_first < 0 || L->rep_first > 2) return fail(ULYS_EINVAL, "rep_first must be 0, 1 or 2");
  if (L->degree > ulys::kMaxDegree) return fail(ULYS_EINVAL, "degree %d exceeds %d", L->degree, ulys::kMaxDegree);
  if (L->hq % L->degree || L->hkv % L->degree)
    return fail(ULYS_EINVAL, "heads (hq %d, hkv %d) must divide by the Ulysses degree %d", L->hq, L->hkv, L->degree);
  if (L->hq % L->hkv) return fail(ULYS_EINVAL, "hq %d must be a multiple of hkv %d", L->hq, L->hkv);
  if ((L->hq / L->degree) % L->groups || (L->hkv / L->degree) % L->groups)
    return fail(ULYS_EINVAL, "groups %d must divide the q heads (%d) and kv heads (%d) per rank", L->groups,
                L->hq / L->degree, L->hkv / L->degree);
  if (L->head_dim != 64 && L->head_dim != 128)
    return fail(ULYS_EUNSUPPORTED, "head_dim %d not built (64, 128)", L->head_dim);
  if (rank < 0 || rank >= L->degree) return fail(ULYS_EINVAL, "rank %d outside [0, %d)", rank, L->degree);
  if (group < -1 || group >= L->groups) return fail(ULYS_EINVAL, "group %d outside [-1, %d)", group, L->groups);
  const long long rows = (long long)L->n_rep + (long long)L->degree * L->s_local;
  if (rows > 0x7fffffffLL) return fail(ULYS_EINVAL, "joint rows %lld too large", rows);
  // the repack kernels index 16-byte chunks of one slot in 32 bits
  const long long hmax = L->hq > L->hkv ? L->hq : L->hkv;
  const long long chunks = (long long)L->batch * rows * (hmax / L->degree / L->groups) * L->head_dim / 8;
  if (chunks >= (1LL << 32)) return fail(ULYS_EINVAL, "slot of %lld 16-byte chunks exceeds 2^32", chunks);
  return ULYS_OK;
}

int check_ptr_array(const void* const* arr, int n, const char* what) {
  if (arr == nullptr) return fail(ULYS_EINVAL, "%s pointer array is NULL", what);
  for (int i = 0; i < n; ++i) {
    if (arr[i] == nullptr) return fail(ULYS_EINVAL, "%s[%d] is NULL", what, i);
    if (!aligned16(arr[i])) return fail(ULYS_EINVAL, "%s[%d] is not 16-byte aligned", what, i);
  }
  return ULYS_OK;
}

int check_ptr(const void* p, const char* what) {
  if (p == nullptr) return fail(ULYS_EINVAL, "%s is NULL", what);
  if (!aligned16(p)) return fail(ULYS_EINVAL, "%s is not 16-byte aligned", what);
  return ULYS_OK;
}

// Repack geometry of one tensor: q (and the output o) or k/v.  With a K/V-only
// prefix (rep_first = 2) q and o carry no replicated rows and k/v carry them
// in front, as with a prefix.
ulys::RepackGeom geom_of(const ulys_layout* L, int rank, int group, bool is_q) {
  ulys::RepackGeom g;
  const int n_rep = (L->rep_first == ULYS_REP_KV_PREFIX && is_q) ? 0 : L->n_rep;
  g.batch = L->batch;
  g.degree = L->degree;
  g.s_local = L->s_local;
  g.n_rep = n_rep;
  g.rep_first = L->rep_first == 0 ? 0 : 1;
  g.rank = rank;
  g.rows = n_rep + L->degree * L->s_local;
  g.shard_rows = n_rep + L->s_local;
  g.head_dim = L->head_dim;
  g.ngroups = group < 0 ? L->groups : 1;
  return g;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(ULYS_EHIP, "HIP: %s", hipGetErrorString(e));
}

// Automatic split of an attention call: none, a key-range split into C runs
// per query tile, or a range split into R runs per (b, head), whichever
// minimises one model of the launch time averaged over calls of 2, 4, 8, 10
// and 16 heads (the choice must not depend on the head count, so that a call
// over a subset of the heads reproduces the full call's bytes), kept only if
// it beats no split by 3%.  Candidates: C in [2, 16] with at least 4 key
// tiles per run; R a multiple of cus / 8 above the query tiles T and up to
// 4T (and 32T, 4096).  Model, in units of one workgroup's sweep over all
// keys (fitted to 45 MI355X measurements of C and R splits at 1500 to 75600
// rows and 2 to 10 heads, D = 128: 2.2% rms error in the speed-up):
//  * workgroups run in rounds of one per CU; a round of a workgroups takes
//    max(0.8, (a / cus)^0.25) of a full one (the device's throughput grows
//    only as the 0.75th power of its busy CUs, with a floor);
//  * a workgroup's share of the keys (1/C, or T/R of a sweep) plus eight key
//    tiles of start-up per piece (one for a key-range run, two for a range);
//  * the merge moves 4C + 2 (C split) or 18 (range split) bytes per output
//    element at 1280 times the per-CU attention rate in bytes per flop.
struct SplitChoice {
  int c;   // key-range runs per query tile (1: none)
  int r;   // range runs per (b, head) (0: none)
};

SplitChoice auto_split(long long batch, long long q_rows, long long kv_rows, int cus) {
  const long long qt = (q_rows + ulys::kAttnRowsPerWorkgroup - 1) / ulys::kAttnRowsPerWorkgroup;
  const double nt = (double)((kv_rows + ulys::kAttnKeysPerTile - 1) / ulys::kAttnKeysPerTile);
  const double units = (double)batch * (double)qt;
  const double kExp = 0.25, kFloor = 0.8, kStartTiles = 8.0, kMergeRate = 1.0 / 1280.0, kGain = 0.97;
  const double kMinTilesPerChunk = 4.0;
  auto rounds = [&](double wgs, double per) {
    const double full = floor(wgs / cus), rest = wgs - full * cus;
    return per * (full + (rest > 0 ? fmax(kFloor, pow(rest / cus, kExp)) : 0.0));
  };
  auto plain = [&](int hq) { return rounds(units * hq, 1.0); };
  auto cost_c = [&](int c, int hq) {
    return rounds(units * c * hq, 1.0 / c + kStartTiles / nt) + hq * units * (4.0 * c + 2.0) * kMergeRate / nt;
  };
  auto cost_r = [&](long long r, int hq) {
    return rounds((double)batch * r * hq, (double)qt / (double)r + 2.0 * kStartTiles / nt) +
           hq * units * 18.0 * kMergeRate / nt;
  };
  static const int kHeads[] = {2, 4, 8, 10, 16};
  constexpr int kNH = sizeof kHeads / sizeof kHeads[0];
  SplitChoice best{1, 0};
  double best_rel = kGain;
  for (int c = 2; c <= ulys::kMaxKeySplits && nt >= c * kMinTilesPerChunk; ++c) {
    double rel = 0.0;
    for (int hq : kHeads) rel += cost_c(c, hq) / plain(hq);
    rel /= kNH;
    if (rel < best_rel) {
      best = SplitChoice{c, 0};
      best_rel = rel;
    }
  }
  const long long step = cus >= 8 ? cus / 8 : 1;
  const long long rmax = std::min<long long>(std::min<long long>(4 * qt, ulys::kMaxRanges),
                                             (long long)ulys::kMaxRangesPerTile * qt);
  for (long long r = (qt / step + 1) * step; r <= rmax; r += step) {
    double rel = 0.0;
    for (int hq : kHeads) rel += cost_r(r, hq) / plain(hq);
    rel /= kNH;
    if (rel < best_rel) {
      best = SplitChoice{1, (int)r};
      best_rel = rel;
    }
  }
  return best;
}

// Compute units of the current device, cached per device.  Threads may race
// to fill an entry; they store the same value, and atomics make that race
// well defined.
constexpr int kCachedDevices = 64;
std::atomic<int> g_cus[kCachedDevices];

int device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  const bool cached = dev >= 0 && dev < kCachedDevices;
  if (cached) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return ULYS_OK;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_status(e);
  if (n < 1) return fail(ULYS_EHIP, "device reports %d compute units", n);
  if (cached) g_cus[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return ULYS_OK;
}

// Validated launch arguments of a pack; nothing is enqueued.
int prepare_pack(const ulys_layout* L, int rank, int group, const void* const* q_shards,
                 const void* const* k_shards, const void* const* v_shards, void* q_slot, void* k_slot,
                 void* v_slot, int qk_dtype, const float* qk_amax, ulys::PackArgs& a) {
  int st = check_layout(L, rank, group);
  if (st) return st;
  if (qk_dtype != ULYS_BF16 && qk_dtype != ULYS_FP8_E4M3) return fail(ULYS_EINVAL, "qk_dtype %d unknown", qk_dtype);
  if ((st = check_ptr_array(q_shards, L->degree, "q_shards"))) return st;
  if ((st = check_ptr_array(k_shards, L->degree, "k_shards"))) return st;
  if ((st = check_ptr_array(v_shards, L->degree, "v_shards"))) return st;
  if ((st = check_ptr(q_slot, "q_slot"))) return st;
  if ((st = check_ptr(k_slot, "k_slot"))) return st;
  if ((st = check_ptr(v_slot, "v_slot"))) return st;
  const bool fp8 = qk_dtype == ULYS_FP8_E4M3;
  if (fp8 && qk_amax == nullptr) return fail(ULYS_EINVAL, "qk_amax is NULL with fp8 q/k");
  if (fp8 && ((uintptr_t)qk_amax & 3u)) return fail(ULYS_EINVAL, "qk_amax is not 4-byte aligned");

  memset(&a, 0, sizeof a);
  for (int t = 0; t < 3; ++t) a.g[t] = geom_of(L, rank, group, t == 0);
  const int heads[3] = {L->hq, L->hkv, L->hkv};
  const void* const* src[3] = {q_shards, k_shards, v_shards};
  void* dst[3] = {q_slot, k_slot, v_slot};
  const int g0 = group < 0 ? 0 : group;
  for (int t = 0; t < 3; ++t) {
    for (int p = 0; p < L->degree; ++p) a.src[t][p] = (const uint16_t*)src[t][p];
    a.dst[t] = dst[t];
    a.heads[t] = heads[t];
    a.gh[t] = heads[t] / L->degree / L->groups;
    a.h0[t] = rank * (heads[t] / L->degree) + g0 * a.gh[t];
    a.fp8[t] = (fp8 && t < 2) ? 1 : 0;
  }
  a.amax = qk_amax;
  return ULYS_OK;
}

// Validated launch arguments of an attention call; nothing is enqueued.
int prepare_attend(int batch, int q_rows, int kv_rows, int hq, int hkv, int head_dim, const void* q, const void* k,
                   const void* v, int qk_dtype, float softmax_scale, const float* qk_amax,
                   const int32_t* key_gaps, const uint32_t* key_mask, int key_splits, void* o, float* lse,
                   ulys::AttnArgs& a) {
  if (batch < 1 || q_rows < 1 || kv_rows < 1 || hq < 1 || hkv < 1)
    return fail(ULYS_EINVAL, "batch, q_rows, kv_rows, hq and hkv must be >= 1");
  if (hq % hkv) return fail(ULYS_EINVAL, "hq %d must be a multiple of hkv %d", hq, hkv);
  if (head_dim != 64 && head_dim != 128) return fail(ULYS_EUNSUPPORTED, "head_dim %d not built (64, 128)", head_dim);
  if (qk_dtype != ULYS_BF16 && qk_dtype != ULYS_FP8_E4M3) return fail(ULYS_EINVAL, "qk_dtype %d unknown", qk_dtype);
  if (batch > 65535 || hq > 65535) return fail(ULYS_EINVAL, "batch and hq must be <= 65535");
  if ((long long)batch * q_rows * hq * head_dim > (1LL << 40) || (long long)batch * kv_rows * hkv * head_dim > (1LL << 40))
    return fail(ULYS_EINVAL, "tensor too large");
  int st;
  if ((st = check_ptr(q, "q"))) return st;
  if ((st = check_ptr(k, "k"))) return st;
  if ((st = check_ptr(v, "v"))) return st;
  if ((st = check_ptr(o, "o"))) return st;
  if (lse != nullptr && ((uintptr_t)lse & 3u)) return fail(ULYS_EINVAL, "lse is not 4-byte aligned");
  const bool fp8 = qk_dtype == ULYS_FP8_E4M3;
  if (fp8 && qk_amax == nullptr) return fail(ULYS_EINVAL, "qk_amax is NULL with fp8 q/k");
  if (fp8 && ((uintptr_t)qk_amax & 3u)) return fail(ULYS_EINVAL, "qk_amax is not 4-byte aligned");
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale))
    return fail(ULYS_EINVAL, "softmax_scale must be finite");
  if (key_splits < -ulys::kMaxRanges || key_splits > ulys::kMaxKeySplits)
    return fail(ULYS_EINVAL, "key_splits %d outside [%d, %d]", key_splits, -ulys::kMaxRanges, ulys::kMaxKeySplits);
  if (key_splits < 0) {
    const long long qtiles = ((long long)q_rows + ulys::kAttnRowsPerWorkgroup - 1) / ulys::kAttnRowsPerWorkgroup;
    if (-(long long)key_splits > qtiles * ulys::kMaxRangesPerTile)
      return fail(ULYS_EINVAL, "%d ranges exceed %d per query tile (%lld tiles)", -key_splits,
                  ulys::kMaxRangesPerTile, qtiles);
  }
  if (key_mask != nullptr) {
    if ((uintptr_t)key_mask & 3u) return fail(ULYS_EINVAL, "key_mask is not 4-byte aligned");
    const long long tiles = ((long long)kv_rows + ulys::kAttnKeysPerTile - 1) / ulys::kAttnKeysPerTile;
    if (tiles > ulys::kMaxMaskTiles)
      return fail(ULYS_EUNSUPPORTED, "a key mask over %d keys exceeds %d", kv_rows,
                  ulys::kMaxMaskTiles * ulys::kAttnKeysPerTile);
  }

  memset(&a, 0, sizeof a);
  if (key_gaps != nullptr) {
    if (batch > ulys::kMaxGapBatch) return fail(ULYS_EINVAL, "key gaps for batch %d > %d", batch, ulys::kMaxGapBatch);
    for (int b = 0; b < batch; ++b) {
      const int g0 = key_gaps[2 * b], g1 = key_gaps[2 * b + 1];
      if (g0 < 0 || g1 < g0 || g1 > kv_rows)
        return fail(ULYS_EINVAL, "key gap [%d, %d) of batch %d outside [0, %d]", g0, g1, b, kv_rows);
      if (g1 - g0 >= kv_rows) return fail(ULYS_EINVAL, "batch %d has no valid key", b);
      a.gap[b][0] = g0;
      a.gap[b][1] = g1;
    }
    a.has_gap = 1;
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.amax = qk_amax;
  a.scale = softmax_scale > 0.0f ? softmax_scale : (float)(1.0 / sqrt((double)head_dim));
  a.batch = batch;
  a.q_rows = q_rows;
  a.kv_rows = kv_rows;
  a.hq = hq;
  a.hkv = hkv;
  a.key_mask = key_mask;
  a.mask_words = (kv_rows + 31) / 32;
  a.splits = key_splits;   // 0: resolved by resolve_splits once every rule has been checked
  return ULYS_OK;
}

// The split of validated arguments: key_splits as given, or (0) the
// automatic choice for `cus` compute units.
void resolve_splits_for(ulys::AttnArgs& a, int cus) {
  if (a.splits < 0) {   // a range split: -splits ranges per (b, head)
    a.ranges = -a.splits;
    a.splits = 1;
    return;
  }
  if (a.splits != 0) return;
  const SplitChoice ch = auto_split(a.batch, a.q_rows, a.kv_rows, cus);
  a.splits = ch.c;
  a.ranges = ch.r;
}

// The split of validated arguments for the current device (the first HIP call
// of an attention call, when the split is automatic).
int resolve_splits(ulys::AttnArgs& a) {
  int cus = 1;
  if (a.splits == 0) {
    const int st = device_cus(&cus);
    if (st) return st;
  }
  resolve_splits_for(a, cus);
  return ULYS_OK;
}

// Workspace bytes a resolved call needs for all its heads in one launch
// (`min_bytes`: for one head per launch; both 0 without a split).
void workspace_need(const ulys::AttnArgs& a, int head_dim, size_t* all_heads, size_t* min_bytes) {
  const ulys::WorkspaceSize w = ulys::attn_workspace_size(a, head_dim);
  *all_heads = w.per_head == 0 ? 0 : w.fixed + w.per_head * (size_t)a.hq;
  *min_bytes = w.per_head == 0 ? 0 : w.fixed + w.per_head;
}

// The caller's workspace must hold at least one head's partials of a split
// call (fewer than all heads: the heads run in several launches).
int check_workspace(const ulys::AttnArgs& a, int head_dim, const void* ws, size_t ws_bytes) {
  size_t all = 0, need = 0;
  workspace_need(a, head_dim, &all, &need);
  if (need == 0) return ULYS_OK;
  if (ws == nullptr || ws_bytes < need)
    return fail(ULYS_EINVAL, "workspace of %zu bytes%s is below the %zu bytes this call needs (%zu for all heads "
                "in one launch; ulys_attend_workspace_bytes)", ws == nullptr ? (size_t)0 : ws_bytes,
                ws == nullptr ? " (NULL)" : "", need, all);
  if ((uintptr_t)ws & 255u) return fail(ULYS_EINVAL, "workspace is not 256-byte aligned");
  return ULYS_OK;
}

// Validated launch arguments of an unpack; nothing is enqueued.
int prepare_unpack(const ulys_layout* L, int rank, int group, const void* o_slot, void* const* o_shards,
                   ulys::UnpackArgs& a) {
  int st = check_layout(L, rank, group);
  if (st) return st;
  if ((st = check_ptr(o_slot, "o_slot"))) return st;
  if ((st = check_ptr_array((const void* const*)o_shards, L->degree, "o_shards"))) return st;
  memset(&a, 0, sizeof a);
  a.g = geom_of(L, rank, group, true);
  a.src = (const uint16_t*)o_slot;
  for (int p = 0; p < L->degree; ++p) a.dst[p] = (uint16_t*)o_shards[p];
  a.heads = L->hq;
  a.gh = L->hq / L->degree / L->groups;
  a.h0 = rank * (L->hq / L->degree) + (group < 0 ? 0 : group) * a.gh;
  return ULYS_OK;
}

}  // namespace

extern "C" {

int ulys_pack(const ulys_layout* L, int rank, int group, const void* const* q_shards,
              const void* const* k_shards, const void* const* v_shards, void* q_slot, void* k_slot,
              void* v_slot, int qk_dtype, const float* qk_amax, void* stream) {
  ulys::PackArgs a;
  const int st = prepare_pack(L, rank, group, q_shards, k_shards, v_shards, q_slot, k_slot, v_slot, qk_dtype,
                              qk_amax, a);
  if (st) return st;
  return hip_status(ulys::launch_pack(a, (hipStream_t)stream));
}

int ulys_amax_bf16(const void* const* tensors, int n_tensors, size_t elems_each, float* amax_out, void* stream) {
  if (n_tensors < 1 || n_tensors > ulys::kMaxAmaxTensors)
    return fail(ULYS_EINVAL, "n_tensors %d outside [1, %d]", n_tensors, ulys::kMaxAmaxTensors);
  int st = check_ptr_array(tensors, n_tensors, "tensors");
  if (st) return st;
  if (elems_each % 8) return fail(ULYS_EINVAL, "elems_each %zu is not a multiple of 8", elems_each);
  if (amax_out == nullptr) return fail(ULYS_EINVAL, "amax_out is NULL");
  if ((uintptr_t)amax_out & 3u) return fail(ULYS_EINVAL, "amax_out is not 4-byte aligned");
  ulys::AmaxArgs a;
  memset(&a, 0, sizeof a);
  for (int i = 0; i < n_tensors; ++i) a.src[i] = (const uint16_t*)tensors[i];
  a.n = n_tensors;
  a.chunks_each = elems_each / 8;
  a.out = (unsigned int*)amax_out;
  return hip_status(ulys::launch_amax(a, (hipStream_t)stream));
}

int ulys_attend_group(int batch, int rows, int hq, int hkv, int head_dim, const void* q, const void* k,
                      const void* v, int qk_dtype, float softmax_scale, const float* qk_amax,
                      const int32_t* key_gaps, void* o, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return ulys_attend_group_ex(batch, rows, rows, hq, hkv, head_dim, q, k, v, qk_dtype, softmax_scale, qk_amax,
                              key_gaps, nullptr, 0, o, lse, workspace, workspace_bytes, stream);
}

int ulys_attend_group_ex(int batch, int q_rows, int kv_rows, int hq, int hkv, int head_dim, const void* q,
                         const void* k, const void* v, int qk_dtype, float softmax_scale, const float* qk_amax,
                         const int32_t* key_gaps, const uint32_t* key_mask, int key_splits, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream) {
  ulys::AttnArgs a;
  int st = prepare_attend(batch, q_rows, kv_rows, hq, hkv, head_dim, q, k, v, qk_dtype, softmax_scale,
                          qk_amax, key_gaps, key_mask, key_splits, o, lse, a);
  if (st || (st = resolve_splits(a)) || (st = check_workspace(a, head_dim, workspace, workspace_bytes))) return st;
  return hip_status(ulys::launch_attn(a, head_dim, qk_dtype == ULYS_FP8_E4M3, workspace, workspace_bytes,
                                      (hipStream_t)stream));
}

int ulys_attend_group_noalloc(int batch, int rows, int hq, int hkv, int head_dim, const void* q, const void* k,
                              const void* v, int qk_dtype, float softmax_scale, const float* qk_amax,
                              const int32_t* key_gaps, void* o, float* lse, void* stream) {
  ulys::AttnArgs a;
  int st = prepare_attend(batch, rows, rows, hq, hkv, head_dim, q, k, v, qk_dtype, softmax_scale, qk_amax, key_gaps,
                          nullptr, 0, o, lse, a);
  if (st || (st = resolve_splits(a))) return st;
  size_t all = 0, need = 0;
  workspace_need(a, head_dim, &all, &need);
  if (need > ulys::kScratchBytes)
    return fail(ULYS_EINVAL, "one head of this call needs %zu bytes of scratch, above the library's static %zu "
                "(use ulys_attend_group with a workspace)", need, ulys::kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = ulys::scratch_address(&ws);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(ulys::launch_attn(a, head_dim, qk_dtype == ULYS_FP8_E4M3, ws, need > 0 ? ulys::kScratchBytes : 0,
                                      (hipStream_t)stream));
}

long long ulys_attend_workspace_bytes(int batch, int q_rows, int kv_rows, int heads, int head_dim, int key_splits,
                                      int compute_units) {
  if (batch < 1 || q_rows < 1 || kv_rows < 1 || heads < 1 || compute_units < 1)
    return fail(ULYS_EINVAL, "batch, q_rows, kv_rows, heads and compute_units must be >= 1");
  if (head_dim != 64 && head_dim != 128) return fail(ULYS_EUNSUPPORTED, "head_dim %d not built (64, 128)", head_dim);
  if (key_splits < -ulys::kMaxRanges || key_splits > ulys::kMaxKeySplits)
    return fail(ULYS_EINVAL, "key_splits %d outside [%d, %d]", key_splits, -ulys::kMaxRanges, ulys::kMaxKeySplits);
  ulys::AttnArgs a;
  memset(&a, 0, sizeof a);
  a.batch = batch;
  a.q_rows = q_rows;
  a.kv_rows = kv_rows;
  a.hq = heads;
  a.splits = key_splits;
  resolve_splits_for(a, compute_units);
  size_t all = 0, one = 0;
  workspace_need(a, head_dim, &all, &one);
  ok();
  return (long long)all;
}

int ulys_unpack(const ulys_layout* L, int rank, int group, const void* o_slot, void* const* o_shards, void* stream) {
  ulys::UnpackArgs a;
  const int st = prepare_unpack(L, rank, group, o_slot, o_shards, a);
  if (st) return st;
  return hip_status(ulys::launch_unpack(a, (hipStream_t)stream));
}

int ulys_rank_pipeline(const ulys_layout* L, int rank, const void* const* q_shards, const void* const* k_shards,
                       const void* const* v_shards, void* q_slots, void* k_slots, void* v_slots, void* o_slots,
                       float* lse, void* const* o_shards, int qk_dtype, const float* qk_amax, float softmax_scale,
                       const int32_t* key_gaps, void* const* events, void* workspace, size_t workspace_bytes,
                       void* stream, void* copy_stream) {
  // Validate everything with group -1 (all groups) before anything is enqueued.
  ulys::PackArgs pk;
  int st = prepare_pack(L, rank, -1, q_shards, k_shards, v_shards, q_slots, k_slots, v_slots, qk_dtype, qk_amax, pk);
  if (st) return st;
  ulys::UnpackArgs up;
  if ((st = prepare_unpack(L, rank, -1, o_slots, o_shards, up))) return st;
  const int G = L->groups;
  const int q_rows = pk.g[0].rows, kv_rows = pk.g[1].rows;
  const int gq = L->hq / L->degree / G, gkv = L->hkv / L->degree / G;
  ulys::AttnArgs at;
  if ((st = prepare_attend(L->batch, q_rows, kv_rows, gq, gkv, L->head_dim, q_slots, k_slots, v_slots, qk_dtype,
                           softmax_scale, qk_amax, key_gaps, nullptr, 0, o_slots, lse, at)))
    return st;
  if (G > ulys::kMaxPipelineGroups)
    return fail(ULYS_EUNSUPPORTED, "pipeline of %d groups exceeds %d", G, ulys::kMaxPipelineGroups);
  if (events == nullptr) return fail(ULYS_EINVAL, "events pointer array is NULL");
  for (int i = 0; i < 3; ++i)
    if (events[i] == nullptr) return fail(ULYS_EINVAL, "events[%d] is NULL", i);
  if ((st = resolve_splits(at)) || (st = check_workspace(at, L->head_dim, workspace, workspace_bytes))) return st;
  const bool fp8 = qk_dtype == ULYS_FP8_E4M3;
  const size_t qk_elem = fp8 ? 1 : 2;
  const size_t elems_q = (size_t)L->batch * q_rows * gq * L->head_dim;
  const size_t elems_kv = (size_t)L->batch * kv_rows * gkv * L->head_dim;
  hipStream_t cs = (hipStream_t)stream, xs = (hipStream_t)copy_stream;

  // The caller's three events.  A stream wait takes the event's state when it
  // is enqueued, so an event may be recorded again once its wait is enqueued:
  // ev_sync carries every single hand-over (start, attention g -> unpack g,
  // done), each waited on right after it is recorded; packs g and g + 1 are
  // outstanding together, so they alternate between ev_pack[0] and [1].
  hipEvent_t ev_sync = (hipEvent_t)events[0];
  hipEvent_t ev_pack[2] = {(hipEvent_t)events[1], (hipEvent_t)events[2]};

  auto pack_g = [&](int g) {
    ulys::PackArgs a = pk;
    for (int t = 0; t < 3; ++t) a.g[t].ngroups = 1;
    for (int t = 0; t < 3; ++t) {
      const size_t bytes = (t == 0 ? elems_q : elems_kv) * (t < 2 ? qk_elem : 2);
      a.dst[t] = (unsigned char*)pk.dst[t] + (size_t)g * bytes;
      a.h0[t] = pk.h0[t] + g * pk.gh[t];
    }
    return ulys::launch_pack(a, xs);
  };
  auto attend_g = [&](int g) {
    ulys::AttnArgs a = at;
    a.q = (const unsigned char*)q_slots + (size_t)g * elems_q * qk_elem;
    a.k = (const unsigned char*)k_slots + (size_t)g * elems_kv * qk_elem;
    a.v = (const unsigned char*)v_slots + (size_t)g * elems_kv * 2;
    a.o = (uint16_t*)o_slots + (size_t)g * elems_q;
    a.lse = lse == nullptr ? nullptr : lse + (size_t)g * L->batch * gq * q_rows;
    return ulys::launch_attn(a, L->head_dim, fp8, workspace, workspace_bytes, cs);
  };
  auto unpack_g = [&](int g) {
    ulys::UnpackArgs a = up;
    a.g.ngroups = 1;
    a.src = (const uint16_t*)o_slots + (size_t)g * elems_q;
    a.h0 = up.h0 + g * up.gh;
    return ulys::launch_unpack(a, xs);
  };

  // copy stream: pack 0, pack 1, [attend 0] unpack 0, pack 2, [attend 1] unpack 1, ...
  // compute stream: [pack g] attend g.  Each group has its own slots, so a
  // pack only has to precede its own attention and an unpack follow it.
  // Attention launches share the workspace in compute-stream order.
  hipError_t e = hipEventRecord(ev_sync, cs);
  if (e == hipSuccess) e = hipStreamWaitEvent(xs, ev_sync, 0);
  for (int g = 0; e == hipSuccess && g < G && g < 2; ++g) {
    e = pack_g(g);
    if (e == hipSuccess) e = hipEventRecord(ev_pack[g & 1], xs);
  }
  for (int g = 0; e == hipSuccess && g < G; ++g) {
    e = hipStreamWaitEvent(cs, ev_pack[g & 1], 0);
    if (e == hipSuccess) e = attend_g(g);
    if (e == hipSuccess) e = hipEventRecord(ev_sync, cs);
    if (e == hipSuccess) e = hipStreamWaitEvent(xs, ev_sync, 0);
    if (e == hipSuccess) e = unpack_g(g);
    if (e == hipSuccess && g + 2 < G) {
      e = pack_g(g + 2);
      if (e == hipSuccess) e = hipEventRecord(ev_pack[g & 1], xs);
    }
  }
  if (e == hipSuccess) e = hipEventRecord(ev_sync, xs);
  if (e == hipSuccess) e = hipStreamWaitEvent(cs, ev_sync, 0);
  return hip_status(e);
}

int ulys_lse_merge(int n_parts, const void* const* o_parts, const float* const* lse_parts, int batch, int rows,
                   int heads, int head_dim, void* o_out, float* lse_out, void* stream) {
  if (n_parts < 1 || n_parts > ulys::kMaxMergeParts)
    return fail(ULYS_EINVAL, "n_parts %d outside [1, %d]", n_parts, ulys::kMaxMergeParts);
  if (batch < 1 || rows < 1 || heads < 1) return fail(ULYS_EINVAL, "batch, rows and heads must be >= 1");
  if (head_dim < 8 || head_dim > 1024 || head_dim % 8)
    return fail(ULYS_EINVAL, "head_dim %d must be a multiple of 8 in [8, 1024]", head_dim);
  if ((long long)batch * rows * heads * head_dim > (1LL << 40)) return fail(ULYS_EINVAL, "tensor too large");
  int st;
  if ((st = check_ptr_array(o_parts, n_parts, "o_parts"))) return st;
  if (lse_parts == nullptr) return fail(ULYS_EINVAL, "lse_parts pointer array is NULL");
  for (int i = 0; i < n_parts; ++i) {
    if (lse_parts[i] == nullptr) return fail(ULYS_EINVAL, "lse_parts[%d] is NULL", i);
    if ((uintptr_t)lse_parts[i] & 3u) return fail(ULYS_EINVAL, "lse_parts[%d] is not 4-byte aligned", i);
    if (lse_out != nullptr && lse_out == lse_parts[i])
      return fail(ULYS_EINVAL, "lse_out must not be one of the lse parts");
  }
  if ((st = check_ptr(o_out, "o_out"))) return st;
  if (lse_out != nullptr && ((uintptr_t)lse_out & 3u)) return fail(ULYS_EINVAL, "lse_out is not 4-byte aligned");
  ulys::MergeArgs a;
  memset(&a, 0, sizeof a);
  for (int i = 0; i < n_parts; ++i) {
    a.o[i] = (const uint16_t*)o_parts[i];
    a.lse[i] = lse_parts[i];
  }
  a.n = n_parts;
  a.out = (uint16_t*)o_out;
  a.lse_out = lse_out;
  a.batch = batch;
  a.rows = rows;
  a.heads = heads;
  a.head_dim = head_dim;
  return hip_status(ulys::launch_lse_merge(a, (hipStream_t)stream));
}

int ulys_attend_splits(int batch, int q_rows, int kv_rows, int compute_units) {
  if (batch < 1 || q_rows < 1 || kv_rows < 1 || compute_units < 1)
    return fail(ULYS_EINVAL, "batch, q_rows, kv_rows and compute_units must be >= 1");
  ok();
  return auto_split(batch, q_rows, kv_rows, compute_units).c;
}

int ulys_attend_ranges(int batch, int q_rows, int kv_rows, int compute_units) {
  if (batch < 1 || q_rows < 1 || kv_rows < 1 || compute_units < 1)
    return fail(ULYS_EINVAL, "batch, q_rows, kv_rows and compute_units must be >= 1");
  ok();
  return auto_split(batch, q_rows, kv_rows, compute_units).r;
}

int ulys_auto_groups(const ulys_layout* L, int compute_units) {
  if (compute_units < 1) return fail(ULYS_EINVAL, "compute_units must be >= 1");
  if (L == nullptr) return fail(ULYS_EINVAL, "layout is NULL");
  ulys_layout one = *L;                 // every layout rule except the group count itself
  one.groups = 1;
  const int st = check_layout(&one, 0, -1);
  if (st) return st;
  // query rows of one call (a K/V-only prefix adds keys, not query rows)
  const long long rows_kv = (long long)L->n_rep + (long long)L->degree * L->s_local;
  const long long rows = (L->rep_first == ULYS_REP_KV_PREFIX ? 0LL : (long long)L->n_rep) +
                         (long long)L->degree * L->s_local;
  const long long hq_rank = L->hq / L->degree, hkv_rank = L->hkv / L->degree;
  // Workgroups of the one-call attention (256 query rows each, times the
  // automatic key-range split, or the range split's runs; the same for every
  // group count; one per CU at a time) and the rounds of CUs they take.
  const SplitChoice ch = auto_split(L->batch, rows, rows_kv, compute_units);
  const long long per_head = ch.r > 0 ? ch.r : (long long)ch.c * ((rows + ulys::kAttnRowsPerWorkgroup - 1) /
                                                                   ulys::kAttnRowsPerWorkgroup);
  const long long wgs = (long long)L->batch * hq_rank * per_head;
  const long long rounds_one = (wgs + compute_units - 1) / compute_units;
  static const int kCandidates[] = {7, 5, 4, 3, 2};
  for (int G : kCandidates) {
    if (hq_rank % G || hkv_rank % G) continue;
    const long long per_call = wgs / G;
    const long long rounds = G * ((per_call + compute_units - 1) / compute_units);
    if (rounds <= rounds_one) {
      ok();
      return G;
    }
  }
  ok();
  return 1;
}

const char* ulys_strerror(int status) {
  switch (status) {
    case ULYS_OK: return "ok";
    case ULYS_EINVAL: return "invalid argument";
    case ULYS_EUNSUPPORTED: return "unsupported configuration";
    case ULYS_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* ulys_last_error(void) { return g_last_error; }

}  // extern "C"
