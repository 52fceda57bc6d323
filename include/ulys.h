/*
 * ulys.h -- C ABI of libulys: one GPU's share of Ulysses sequence-parallel
 * attention on MI355X (gfx950).
 *
 * Three steps make the path, each a call below:
 *   ulys_pack          shards -> per-head-group receive slots (+ optional e4m3 q/k)
 *   ulys_attend_group  dense non-causal attention + log-sum-exp on one slot
 *   ulys_unpack        output slot -> output shards
 * plus ulys_rank_pipeline (the three steps for every head group of a rank,
 * repack overlapping attention on a second stream), ulys_lse_merge (merge of
 * partial results over key blocks, for ring / hybrid parallelism), ulys_amax_bf16
 * (per-tensor fp8 scale source), ulys_attend_group_ex (different query and key
 * lengths, key masks, an explicit work split), ulys_attend_splits /
 * ulys_attend_ranges / ulys_auto_groups / ulys_attend_workspace_bytes (the
 * automatic choices and the workspace size, host-only), ulys_attend_group_noalloc
 * (attention for callers that cannot allocate), ulys_strerror and
 * ulys_last_error.
 *
 * Conventions shared by every call
 *   - Tensors are caller-owned device memory, dense, row-major, with the
 *     shapes stated per call; bf16 is IEEE bfloat16, fp8 is OCP e4m3fn (one
 *     byte per element).  Every device pointer must be 16-byte aligned.
 *   - Arrays of pointers and key gaps are host memory, read only during the
 *     call; the caller may reuse them on return.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on it; none synchronises, allocates device memory, or keeps state
 *     between calls.  Scratch memory (the attention workspace) and the
 *     pipeline's events are the caller's, passed in like the tensors
 *     (sglang PR #43521, "Buffers": the caller's pool holds every buffer of
 *     the path).  The only state is the text behind ulys_last_error, a
 *     cache of each device's compute-unit count, and the static scratch
 *     array of ulys_attend_group_noalloc (with its per-device address).
 *   - All validation happens before anything is enqueued.  On failure the
 *     call returns a negative ulys_status, enqueues nothing, and
 *     ulys_last_error() describes the first violated rule.
 *   - The all-to-all of the method is modelled as a local permutation: the
 *     P "shards" below are the P ranks' inputs, all resident on this GPU.
 *
 * Glossary: B batch, P Ulysses degree, S_l sharded rows per rank, R
 * replicated text rows, rows = R + P*S_l, Hq/Hkv model heads, G head groups
 * per rank, Gq = Hq/(P*G), Gkv = Hkv/(P*G), D head_dim.
 */
#ifndef ULYS_H
#define ULYS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ULYS_OK = 0,
  ULYS_EINVAL = -1,        /* an argument breaks a rule stated below */
  ULYS_EUNSUPPORTED = -2,  /* valid but not built: head_dim not 64/128, fp8 V */
  ULYS_EHIP = -3           /* the HIP runtime refused a launch */
} ulys_status;

typedef enum {
  ULYS_BF16 = 0,
  ULYS_FP8_E4M3 = 1        /* OCP e4m3fn codes, one per-tensor scale each for q and k */
} ulys_dtype;

/* ulys_layout.rep_first values */
typedef enum {
  ULYS_REP_SUFFIX = 0,     /* replicated rows behind the shard rows, in q, k and v */
  ULYS_REP_PREFIX = 1,     /* replicated rows in front of the shard rows, in q, k and v */
  ULYS_REP_KV_PREFIX = 2   /* replicated rows in front in k and v only; q and o have none */
} ulys_rep_mode;

/*
 * Layout of one Ulysses attention call, as every rank sees it.
 *
 * Each of the P shards of q (resp. k, v) is [B, R + S_l, Hq (resp. Hkv), D]
 * bf16.  With R > 0 the replicated rows sit in front of the shard rows when
 * rep_first = 1 (a replicated prefix) and behind them when rep_first = 0
 * (a replicated suffix).  Source: sglang multimodal_gen attention layer.py,
 * USPAttention.forward (num_replicated_prefix / num_replicated_suffix) and
 * sglang PR #43521 "Layouts" (q/k/v as [batch, s_local, heads, head_dim],
 * GQA, replicated prefix or suffix).
 *
 * rep_first = 2 (ULYS_REP_KV_PREFIX) is cross-attention with a replicated
 * K/V-only prefix (sglang layer.py _forward_with_replicated_kv_prefix: q is
 * sequence-sharded with no replicated part; k/v carry the replicated prefix
 * followed by the shard rows, which line up with q's sharding; sglang PR
 * #43521 "Layouts", a K/V-only prefix).  Then q shards and o shards are
 * [B, S_l, Hq, D] and k/v shards [B, R + S_l, Hkv, D]; the q and o slots
 * hold P*S_l rows and the k/v slots R + P*S_l rows.
 *
 * Rules (ULYS_EINVAL otherwise): batch, degree, s_local, hq, hkv, groups >= 1;
 * n_rep >= 0; rep_first in {0, 1, 2}; P | Hq and P | Hkv (flashdreams cp.py,
 * ContextParallelAttention._impl_ulysses: heads must divide by the CP size);
 * Hkv | Hq (GQA); G | Hq/P and G | Hkv/P (sglang PR #43521, "Automatic group
 * count": a group count must divide the q and k/v heads per rank); a q slot
 * batch * rows * (Hq/(P*G)) * head_dim * 2 bytes holds fewer than 2^32 16-byte
 * chunks (64 GiB; the repack kernels index chunks in 32 bits).
 * head_dim in {64, 128} (ULYS_EUNSUPPORTED otherwise).
 */
typedef struct ulys_layout {
  int32_t batch;
  int32_t degree;     /* P */
  int32_t s_local;    /* S_l */
  int32_t n_rep;      /* R, 0 = no replicated rows */
  int32_t rep_first;  /* ulys_rep_mode: 1 prefix, 0 suffix, 2 K/V-only prefix */
  int32_t hq;
  int32_t hkv;
  int32_t head_dim;   /* D */
  int32_t groups;     /* G */
} ulys_layout;

/*
 * ulys_pack -- fill the receive slots of head group `group` of rank `rank`.
 *
 * Source: sglang PR #43521, "Receive slots" (per head group one contiguous
 * [batch, rows, group_heads, head_dim] tensor in the order attention reads)
 * and "Layouts" (replicated rows stay out of the exchange; each rank places
 * its own copy); flashdreams cp.py _impl_ulysses (rank r receives heads
 * [r*H/P, (r+1)*H/P), sharded rows source-rank-major); sglang layer.py
 * _forward_with_replicated_prefix (replicated rows sliced to the rank's
 * heads, q and k/v separately, then joined in front).
 *
 *   slot[b, t, j, :] = J_r[b, t, h0 + j, :],  h0 = r*H/P + g*H/(P*G)
 * where J_r is the joint sequence of rank r: prefix [rep(r) | shard rows of
 * ranks 0..P-1], suffix [shard rows of ranks 0..P-1 | rep(r)], rep(r) being
 * shard r's copy of the replicated rows.  Groups take contiguous head blocks.
 *
 * With a K/V-only prefix, J_r of q is the shard rows of ranks 0..P-1 alone
 * and J_r of k/v the prefix form.
 *
 * q_shards/k_shards/v_shards: host arrays of P device pointers (layout above).
 * q_slot: [B, rows_q, Gq, D], k_slot/v_slot: [B, rows_kv, Gkv, D], where
 * rows_kv = R + P*S_l and rows_q = rows_kv, or P*S_l with a K/V-only prefix.  group = -1
 * packs all G groups at once into G consecutive slots ([G][B, rows, Gh, D]).
 * q_slot and k_slot hold bf16 when qk_dtype = ULYS_BF16 and e4m3fn codes
 * (1 byte per element) when qk_dtype = ULYS_FP8_E4M3; v_slot is always bf16.
 *
 * fp8 (LightX2V PR "Add optimized Ulysses attention path": fp8 payloads
 * travel with a separate scale): qk_amax is a device pointer to two floats
 * {max|q|, max|k|} over all shards (ulys_amax_bf16 writes them); the kernel
 * forms inv = 448 / amax in float32 (1 if amax = 0) and writes
 * e4m3fn_rne(clamp(float32(x) * inv, -448, 448)).  qk_amax is ignored
 * (may be NULL) for ULYS_BF16.
 */
int ulys_pack(const ulys_layout* layout, int rank, int group,
              const void* const* q_shards, const void* const* k_shards,
              const void* const* v_shards,
              void* q_slot, void* k_slot, void* v_slot,
              int qk_dtype, const float* qk_amax, void* stream);

/*
 * ulys_lse_merge -- merge the partial results of attention over disjoint key
 * blocks into the result over all of them.
 *
 * Source: flashdreams cp.py, ContextParallelAttention, ring path (ring
 * attention over the CP ranks' key blocks: the running result takes in each
 * step's output with a logistic weight of the LSE difference and its LSE
 * becomes the log of the summed exponentials, optionally in float32); the
 * Ulysses + ring hybrid of sglang's USPAttention uses the same merge across
 * its ring dimension.
 *
 * For every b, head h, row i:  L = ln sum_p exp(lse_p),
 *   o_out = sum_p exp(lse_p - L) * o_p,  lse_out = L
 * (the closed form of absorbing the parts one after the other), in float32,
 * o_out rounded to bf16 (nearest even).  A part with lse = -inf (no valid key
 * in its block) has weight 0; a row whose parts are all -inf gets o = 0 and
 * lse = -inf.
 *
 * o_parts: host array of n_parts device pointers, each [B, rows, heads, D]
 * bf16 (the o of ulys_attend_group); lse_parts: host array of n_parts device
 * pointers, each [B, heads, rows] float32 (its lse).  o_out: [B, rows, heads,
 * D] bf16, may be one of o_parts (each element is read before it is written);
 * lse_out: [B, heads, rows] float32 or NULL, not one of lse_parts.
 * Rules (ULYS_EINVAL otherwise): 1 <= n_parts <= 16; batch, rows, heads >= 1;
 * head_dim a multiple of 8 in [8, 1024]; o pointers 16-byte aligned, lse
 * pointers 4-byte aligned, none NULL (lse_out may be).
 */
int ulys_lse_merge(int n_parts, const void* const* o_parts, const float* const* lse_parts,
                   int batch, int rows, int heads, int head_dim,
                   void* o_out, float* lse_out, void* stream);

/*
 * ulys_auto_groups -- the head-group count for ulys_rank_pipeline on this GPU.
 *
 * Source: sglang PR #43521, "Automatic group count" (the largest of 7, 5, 4,
 * 3 and 2 that divides the q and k/v heads per rank while each group's call
 * still fills the GPU; otherwise no split -- calls too small to fill the
 * device cost more than the overlap saves).
 *
 * The fill test is MI355X's, re-measured for this library's attention (one
 * 256-row workgroup per CU at a time, so a call runs in rounds of
 * compute_units workgroups and a partial round costs nearly a full one): G is
 * accepted when G calls take no more rounds than the one call over all the
 * rank's heads, i.e. G * ceil(W / G / cus) <= ceil(W / cus) with
 * W = batch * (Hq/P) * ceil(rows_q / 256) * C, C the automatic key-range
 * split of the shape (ulys_attend_splits), or W = batch * (Hq/P) * R under
 * an automatic range split R (ulys_attend_ranges); neither depends on the
 * head count, so they are the same for every G.  Returns the count (>= 1; 1 = keep
 * the sequential single call); layout->groups is ignored.
 * Rules: the layout rules with groups = 1; compute_units >= 1 (ULYS_EINVAL).
 */
int ulys_auto_groups(const ulys_layout* layout, int compute_units);

/*
 * ulys_amax_bf16 -- amax_out[0] = max |x| over n_tensors bf16 device arrays
 * of elems_each elements each (the per-tensor fp8 scale source; exact,
 * independent of order).  amax_out is a device float, overwritten.
 *
 * Source: LightX2V PR "Add optimized Ulysses attention path", review of the
 * fp8 communication records (the fp8 payload and its scale travel as two
 * tensors, and the receiver dequantises with the scale); the pages give no
 * scale formula, and this library reads it as one scale per tensor over all
 * shards, amax / 448 (the largest e4m3fn magnitude), so that the largest
 * element maps to the largest code.
 * Rules: n_tensors >= 1, every pointer non-NULL and 16-byte aligned,
 * elems_each a multiple of 8 (ULYS_EINVAL otherwise).
 */
int ulys_amax_bf16(const void* const* tensors, int n_tensors, size_t elems_each,
                   float* amax_out, void* stream);

/*
 * ulys_attend_group -- dense non-causal softmax attention with LSE on one
 * head group's slots.
 *
 * Source: flashdreams cp.py torch_sdpa_cudnn / torch_sdpa_flash (attention
 * that returns the log-sum-exp); sglang PR #43521 "Receive slots"
 * (attend(q, k, v) on views of the slot); sglang layer.py LocalAttention
 * (key mask = zero weight for masked keys; GQA repeats each k/v head
 * Hq/Hkv times) and USPAttention.forward (a contiguous pad span
 * [pad_start, pad_end) of masked keys); UlyssesAttention.__init__ (default
 * scale head_dim^-1/2).
 *
 * For each b, q head h (kv head h / (hq/hkv)), row i, over the valid keys J
 * (those outside [key_gaps[2b], key_gaps[2b+1])):
 *   s_ij = c * <q_i, k_j>,  o_i = sum_J softmax(s)_ij v_j,  lse_i = ln sum_J exp(s_ij)
 * c = softmax_scale (<= 0 selects head_dim^-1/2), times q_scale * k_scale
 * (scale = amax / 448, or 1 if amax = 0, from qk_amax) for fp8 q/k,
 * all in float32.  Query rows inside the gap are computed like any other
 * row (the mask is on keys only).
 *
 * q: [B, rows, hq, D], k/v: [B, rows, hkv, D]; q/k bf16 or e4m3fn codes
 * (qk_dtype), v bf16.  o: [B, rows, hq, D] bf16 (round to nearest even).
 * lse: [B, hq, rows] float32, natural log, or NULL to skip it.
 * key_gaps: host int32 [B][2] half-open masked key range per batch, or NULL
 * for none; 0 <= start <= end <= rows and end - start < rows (a batch
 * without a valid key is ULYS_EINVAL), B <= 256 when given.
 * Rules: rows >= 1, hq % hkv == 0, head_dim in {64, 128}.  Each head's
 * result depends only on that head's data: calling on a head subset gives
 * the same bytes for those heads as the full call.
 *
 * Key-range split (automatic, see ulys_attend_splits): when the query tiles
 * of a call are too few to keep every compute unit busy, each (b, head,
 * 256-row query tile) is computed as C workgroups over C contiguous runs of
 * its 64-key tiles, each writing an fp32 partial (o, lse); a second kernel
 * combines them in run order with the log-sum-exp weights.  C depends on
 * (batch, rows, the device's compute units) only, so the head-subset rule
 * above still holds.
 *
 * Workspace: the partials of a split live in `workspace`, caller-owned
 * device memory of `workspace_bytes` bytes, 256-byte aligned.
 * ulys_attend_workspace_bytes gives the size for all heads in one launch (0
 * when the call takes no split; then workspace may be NULL).  A smaller
 * workspace that still holds one head's partials (the size for heads = 1)
 * runs the heads in several launches, with the same bytes; below that the
 * call is ULYS_EINVAL.  The call overwrites the workspace; calls that share
 * one must be ordered (one stream, or events).
 *
 * Range split (automatic, see ulys_attend_ranges): the (query
 * tile, key tile) pairs of each (b, head), taken query tile by query tile,
 * are cut into R near-equal runs, one workgroup each, so that a call's
 * workgroups fill whole rounds of CUs with less than a query tile each.  A
 * query tile inside one run is written directly; the pieces of a tile cut
 * by run ends write fp32 partials (same workspace) that a second kernel
 * combines in run order with the log-sum-exp weights.  R depends on (batch,
 * rows, compute units) only, so the head-subset rule holds here too.  Its
 * partials live in the same workspace.
 */
int ulys_attend_group(int batch, int rows, int hq, int hkv, int head_dim,
                      const void* q, const void* k, const void* v, int qk_dtype,
                      float softmax_scale, const float* qk_amax,
                      const int32_t* key_gaps, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * ulys_attend_group_noalloc -- ulys_attend_group for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments without the
 * workspace, the same kernels and the same bytes.
 *
 * The split partials live in a static device array of the library, 128 MiB
 * per GPU, held from the first call on that GPU until the process ends; the
 * call itself allocates nothing.  A call whose heads need more than the
 * array runs them in several launches (as a small
 * workspace does for ulys_attend_group); one whose single head needs more is
 * ULYS_EINVAL with nothing enqueued.  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (different streams, no ordering
 * between them) race and may return wrong results; calls ordered on one
 * stream are safe.  Nothing in the array has to start at zero.
 */
int ulys_attend_group_noalloc(int batch, int rows, int hq, int hkv, int head_dim,
                              const void* q, const void* k, const void* v, int qk_dtype,
                              float softmax_scale, const float* qk_amax,
                              const int32_t* key_gaps, void* o, float* lse, void* stream);

/*
 * ulys_attend_group_ex -- ulys_attend_group with query and key sequences of
 * different lengths and an optional arbitrary key mask.
 *
 * Source: sglang layer.py _forward_with_replicated_kv_prefix (attention of the
 * gathered q rows over [replicated K/V prefix | gathered k/v rows]: more keys
 * than queries); sglang PR #43521 path table, "key mask / tail padding" (a
 * gathered key mask, attended with varlen FA or SDPA) and layer.py
 * build_varlen_mask_meta (a [B, S] boolean key mask; masked keys take no part
 * in any row's softmax) and LocalAttention (masked keys get zero weight).
 *
 * As ulys_attend_group, with q, o: [B, q_rows, hq, D], k, v: [B, kv_rows,
 * hkv, D], lse: [B, hq, q_rows], key_gaps ranges inside [0, kv_rows], and
 * the valid keys of batch b being those outside its gap whose bit is set in
 * key_mask: a device array of B * ceil(kv_rows / 32) uint32 words, key j of
 * batch b valid iff bit (j % 32) of word [b * ceil(kv_rows/32) + j / 32] is 1
 * (bits for j >= kv_rows are ignored), or NULL for all keys valid.  Key tiles
 * (64 keys) without a valid key are skipped.  A (b, row) left without any
 * valid key by the mask gets o = 0 and lse = -inf (the mask is device data,
 * so this cannot be rejected up front).  Query rows are never masked.
 * Rules: as ulys_attend_group with q_rows, kv_rows >= 1; key_mask 4-byte
 * aligned; with a key mask kv_rows <= 262144 (ULYS_EUNSUPPORTED otherwise).
 * key_splits: 0 = automatic (ulys_attend_splits, else ulys_attend_ranges,
 * of the device), 1 = no split, 2..16 = that many key-range runs per query
 * tile, -R = a range split into R runs per (b, head) (1 <= R <= 4096 and
 * R <= 32 x the query tiles ceil(q_rows / 256)); anything else ULYS_EINVAL.
 * Runs are near-equal shares of the processed key tiles (of the query-tile
 * by key-tile pairs for -R), and a run without tiles contributes nothing.
 * ulys_attend_group(B, rows, ...) equals ulys_attend_group_ex(B, rows, rows,
 * ..., key_mask = NULL, key_splits = 0, ...), and a mask that marks exactly
 * the keys outside the gaps gives the same bytes as the gaps (at equal
 * key_splits).  workspace / workspace_bytes as for ulys_attend_group (sized
 * by ulys_attend_workspace_bytes with the same key_splits).
 */
int ulys_attend_group_ex(int batch, int q_rows, int kv_rows, int hq, int hkv, int head_dim,
                         const void* q, const void* k, const void* v, int qk_dtype,
                         float softmax_scale, const float* qk_amax,
                         const int32_t* key_gaps, const uint32_t* key_mask, int key_splits,
                         void* o, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * ulys_attend_workspace_bytes -- device workspace bytes that an attention call
 * of this shape needs for all `heads` of it in one launch.
 *
 * Source: sglang PR #43521, "Buffers" (the caller's pool holds every buffer
 * of the attention path, sized once per shape); the workspace holds the
 * partial results of a split launch (ulys_attend_group), combined by their
 * log-sum-exp as in flashdreams cp.py, ContextParallelAttention, ring path.
 *
 * key_splits as for ulys_attend_group_ex (0 = the automatic choice, which
 * depends on compute_units: pass the device's compute-unit count,
 * hipDeviceAttributeMultiprocessorCount).  Returns the byte count (>= 0; 0:
 * no split, no workspace), or a negative ulys_status: ULYS_EINVAL if an
 * argument is < 1 or key_splits is out of range, ULYS_EUNSUPPORTED for
 * head_dim not 64/128.  Host-only: enqueues nothing.  With heads = 1 it
 * gives the smallest workspace the call accepts.
 */
long long ulys_attend_workspace_bytes(int batch, int q_rows, int kv_rows, int heads, int head_dim,
                                      int key_splits, int compute_units);

/*
 * ulys_attend_splits -- the automatic key-range split of an attention call.
 *
 * Source: the per-rank attention over the full gathered sequence (sglang
 * PR #43521, "Receive slots"; flashdreams cp.py torch_sdpa_*) is one launch
 * whose workgroup count is fixed by the shape; the split and its merge are
 * the log-sum-exp combination of partial attentions over disjoint key sets
 * (flashdreams cp.py, ContextParallelAttention._impl_ring).
 *
 * Returns the run count C >= 1 that ulys_attend_group uses for
 * (batch, q_rows, kv_rows) on a device with compute_units CUs (1: no
 * key-range split).  One model chooses among no split, C in [2, 16] (each
 * run >= 4 key tiles) and the range split of ulys_attend_ranges: the choice
 * minimising the modelled launch time averaged over calls of 2, 4, 8, 10 and
 * 16 heads, if it beats no split by 3%.  The model: workgroups run in rounds
 * of one per CU and a round of a workgroups takes max(0.8, (a / cus)^0.25)
 * of a full one (the device's throughput grows as the 0.75th power of its
 * busy CUs); a workgroup does its share of the keys plus eight key tiles of
 * start-up per piece; the merge moves 4C + 2 (or, for a range split, 18)
 * bytes per output element.  Host-only: enqueues nothing.  A negative
 * status (ULYS_EINVAL) if an argument is < 1.
 */
int ulys_attend_splits(int batch, int q_rows, int kv_rows, int compute_units);

/*
 * ulys_attend_ranges -- the automatic range split of an attention call.
 *
 * Source: as ulys_attend_splits (one launch per call whose workgroup count
 * the shape fixes; partial attentions over disjoint key sets combined by
 * their log-sum-exp).
 *
 * Returns the run count R > 0 that ulys_attend_group uses for (batch,
 * q_rows, kv_rows) on compute_units CUs, or 0 when the same model (see
 * ulys_attend_splits) chooses no split or a key-range split.  Candidates are
 * the multiples of compute_units / 8 above the query tiles
 * T = ceil(q_rows / 256) and up to 4T; a range does T / R of a key sweep plus
 * two pieces' start-up.  Host-only: enqueues nothing.  A negative status
 * (ULYS_EINVAL) if an argument is < 1.
 */
int ulys_attend_ranges(int batch, int q_rows, int kv_rows, int compute_units);

/*
 * ulys_unpack -- inverse of ulys_pack for the output of (rank, group).
 *
 * Source: flashdreams cp.py _impl_ulysses (output all-to-all restores the
 * sequence shards); sglang layer.py _forward_with_replicated_prefix
 * (the replicated rows' output is all-gathered over heads, so every rank
 * gets it) and sglang PR #43521 "Layouts" (output returns in the caller's
 * row order).
 *
 * o_slot: [B, rows_q, Gq, D] bf16 (group = -1: [G][B, rows_q, Gq, D]).
 * o_shards: host array of P device pointers, each [B, R + S_l, Hq, D] bf16
 * ([B, S_l, Hq, D] with a K/V-only prefix);
 * writes heads h0..h0+Gq of every shard: shard rows of rank p from their
 * joint rows, replicated rows into every shard.  Other heads are untouched.
 */
int ulys_unpack(const ulys_layout* layout, int rank, int group,
                const void* o_slot, void* const* o_shards, void* stream);

/*
 * ulys_rank_pipeline -- one rank's whole path, head group by head group, with
 * the repack of neighbouring groups overlapping each group's attention.
 *
 * Source: sglang PR #43521, "Motivation" and "Receive slots" (split the
 * heads into groups and run exchange-in(g+1) and exchange-out(g-1) on a
 * second stream while group g attends, each group in its own receive slot,
 * with events between the streams; the result must be the sequential
 * exchange's, bit for bit) and "Host cost" (no host synchronisation inside
 * the loop).
 *
 * Equivalent to, for g = 0 .. G-1 in order:
 *   ulys_pack(layout, rank, g, ...) into slot g,
 *   ulys_attend_group_ex(B, rows_q, rows_kv, Gq, Gkv, D, slot g ..., key_splits 0, o slot g, lse g),
 *   ulys_unpack(layout, rank, g, o slot g, o_shards)
 * and byte-identical to it.  q/k/v/o_slots hold G consecutive slots
 * ([G][B, rows, Gh, D], the group = -1 layout of ulys_pack); lse is
 * [G][B, Gq, rows_q] float32 or NULL.  Shards, qk_dtype, qk_amax,
 * softmax_scale and key_gaps as for ulys_pack / ulys_attend_group.
 *
 * Streams: attention runs on `stream`, packs and unpacks on `copy_stream`
 * (pack(g+2) and unpack(g) follow attention g there).  The call orders the
 * copy stream after work already enqueued on `stream`, and work enqueued on
 * `stream` after the call after the last unpack, so the caller synchronises
 * on `stream` alone.  Passing the same stream twice runs everything in order
 * on it.  Every rule of the three calls is checked before anything is
 * enqueued; G <= 64 (ULYS_EUNSUPPORTED otherwise).
 *
 * events: host array of 3 hipEvent_t that the caller created (any flags;
 * hipEventDisableTiming is the cheapest) and owns; the call records them on
 * the two streams and makes each stream wait on them (a stream wait takes the
 * event's state when it is enqueued), and creates or destroys none, so the
 * same three may serve every call.  workspace / workspace_bytes: the
 * attention workspace (ulys_attend_group) for Gq heads at
 * (B, rows_q, rows_kv), shared by the G attention launches in stream order.
 */
int ulys_rank_pipeline(const ulys_layout* layout, int rank,
                       const void* const* q_shards, const void* const* k_shards,
                       const void* const* v_shards,
                       void* q_slots, void* k_slots, void* v_slots, void* o_slots,
                       float* lse, void* const* o_shards,
                       int qk_dtype, const float* qk_amax, float softmax_scale,
                       const int32_t* key_gaps, void* const* events,
                       void* workspace, size_t workspace_bytes,
                       void* stream, void* copy_stream);

/* Static text for a ulys_status value. */
const char* ulys_strerror(int status);

/* Text naming the rule the last failed call on this thread broke ("" if none). */
const char* ulys_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ULYS_H */
