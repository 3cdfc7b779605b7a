/*
 * oxa.h - BF16 attention over a paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Four operations make up the path:
 *
 *   oxa_paged_append_rope  fused NeoX RoPE on q/k + append of (k, v) into
 *                          exclusively owned KV pages (oxa_paged_append:
 *                          the same append without RoPE)
 *   oxa_paged_decode       paged batch decode (MHA / GQA / MQA), optionally
 *                          split-K over explicit KV partitions with an f32
 *                          partial workspace and a log-sum-exp merge
 *   oxa_ragged_prefill     causal (or full) prefill over packed ragged K/V
 *   oxa_paged_prefill      causal (or full) prefill over paged K/V (both may
 *                          split a small call's keys over more compute
 *                          units, given an optional workspace)
 *
 * and two standalone operations: the attention-state merge
 * (oxa_merge_states, oxa_merge_state_pair), which combines the (output, lse)
 * states of disjoint key sets as split-K decode does internally and cascade /
 * shared-prefix attention does across calls, and NeoX RoPE on q and k at
 * explicit positions (oxa_rope_neox, oxa_rope_llama31).
 *
 * The operator contracts follow the "FlashInfer parity matrix" page (sections
 * "Admitted attention matrix", "Dispatch limits", "Paged KV ownership
 * difference", "Domain coverage") and the runtime rules on the "Oxide Infer"
 * README page (sections "One execution model" and "Providers": caller-selected
 * stream, typed read and write regions, checked span / alignment / alias /
 * capacity, explicit workspace, typed device-status failures, no tuning or
 * silent fallback at enqueue).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Types.   bf16 tensors are passed as uint16_t bit patterns; indices are int32.
 * Memory.  Every tensor pointer is a DEVICE pointer (hipMalloc'd or a torch
 *          CUDA tensor), except where a comment says "host".  The caller owns
 *          all memory.  The library allocates nothing, frees nothing, keeps no
 *          pointer after the call returns and keeps no state between calls
 *          apart from a per-device cache of the compute-unit count and, for
 *          oxa_paged_decode_noalloc only, its static per-GPU scratch array.
 * Stream.  Work is enqueued on `stream` (0 = the null stream) and the call
 *          returns without synchronising.  Buffers must stay valid, and inputs
 *          unmodified, until that work completes.
 * Errors.  Host-detectable contract violations (null pointer, unsupported
 *          shape, misalignment, overlapping regions, short workspace) return
 *          an OXA_ERR_* code at once and enqueue NOTHING.  Data-dependent
 *          violations (bad indptr, page ids outside the pool, lengths beyond
 *          the declared maxima, refcount != 1, positions beyond capacity) are
 *          reported through the `status` array on the stream; kernels never
 *          read or write outside the regions the arguments describe, whatever
 *          the metadata holds.  Rows of a sequence whose status is non-zero
 *          are unspecified.
 *          OXA_ERR_LAUNCH is the one exception to "nothing enqueued": an
 *          operation of two kernels (append check + writer, split-K decode +
 *          merge, key-split prefill + merge) whose second launch is refused
 *          leaves the first one enqueued; its outputs and status are then
 *          unspecified.  Host validation rules out every launch shape the
 *          runtime could refuse, so this code means a failing runtime.
 * Domain.  head_dim must be 128 and page_size 16 (OXA_ERR_UNSUPPORTED else).
 *          Head grouping: num_qo_heads % num_kv_heads == 0; q head h reads
 *          kv head h / (num_qo_heads / num_kv_heads).
 * Layouts. K and V live in two pools of num_pages pages each:
 *            OXA_LAYOUT_NHD: [num_pages][page_size][num_kv_heads][head_dim]
 *            OXA_LAYOUT_HND: [num_pages][num_kv_heads][page_size][head_dim]
 * Pages.   Sequence b lists its physical pages in
 *          page_indices[page_indptr[b] .. page_indptr[b+1]); its logical token
 *          j is slot j % 16 of page page_indices[page_indptr[b] + j / 16].
 *          Pages may appear in any physical order, and attention may read a
 *          page listed by several sequences.  A sequence may list more pages
 *          than its length needs; attention reads only the first
 *          ceil(len / 16).  num_page_entries is the length of page_indices.
 * Alignment. Every bf16 tensor and the workspace must be 16-byte aligned.
 * Softmax. sm_scale must be finite and >= 0 (0 weighs every visible key
 *          alike: the output is the mean of their V rows and lse = ln(count);
 *          masked keys and tail slots still weigh nothing).  f32 running max / sum /
 *          accumulator; outputs rounded to bf16 (nearest-even).  lse
 *          (optional, may be NULL) is the natural-log log-sum-exp of the
 *          scaled scores of each (query row, q head).
 */
#ifndef OXA_H
#define OXA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OXA_ABI_VERSION 8
#define OXA_PAGE_SIZE 16
#define OXA_HEAD_DIM 128

typedef enum { OXA_LAYOUT_NHD = 0, OXA_LAYOUT_HND = 1 } oxa_layout;

/* element type of attention states (oxa_merge_*) */
typedef enum { OXA_DTYPE_BF16 = 0, OXA_DTYPE_F32 = 1 } oxa_dtype;

typedef enum {
  OXA_OK = 0,
  /* returned by the call itself; nothing was enqueued */
  OXA_ERR_NULL = 1,          /* a required pointer is NULL */
  OXA_ERR_UNSUPPORTED = 2,   /* head_dim != 128, page_size != 16, unknown layout or dtype */
  OXA_ERR_SHAPE = 3,         /* a count or scalar is out of range, or Hq % Hkv != 0 */
  OXA_ERR_ALIGN = 4,         /* a bf16 tensor or the workspace is not 16-byte aligned */
  OXA_ERR_ALIAS = 5,         /* an output region overlaps an input or another output */
  OXA_ERR_WORKSPACE = 6,     /* workspace NULL or smaller than the size query returns */
  OXA_ERR_LAUNCH = 7,        /* the HIP runtime refused a kernel launch (see Errors) */
  OXA_ERR_SCRATCH_LIMIT = 8, /* oxa_paged_decode_noalloc: the partial states need more than
                                OXA_DECODE_SCRATCH_BYTES */
  /* written to status[] on the stream by the kernels */
  OXA_DEV_PAGE_RANGE = 16,   /* a needed page id is outside [0, num_pages) */
  OXA_DEV_INDPTR = 17,       /* indptr out of order / beyond its array, or too few pages */
  OXA_DEV_SEQ_LEN = 18,      /* a length is < 1 (where required) or above its declared max */
  OXA_DEV_CAUSAL = 19,       /* causal with more query rows than keys */
  OXA_DEV_NOT_EXCLUSIVE = 20,/* an append target page has refcount != 1 */
  OXA_DEV_CAPACITY = 21,     /* an append position is < 0 or beyond the listed pages */
  OXA_DEV_BATCH_INDEX = 22   /* an append token names a sequence outside [0, batch) */
} oxa_status;

/* ABI version compiled into the library (OXA_ABI_VERSION). */
int32_t oxa_abi_version(void);

/* Static, human-readable name of a status code ("OXA_OK", ...; "unknown"). */
const char* oxa_status_string(int32_t code);

/*
 * Fused NeoX RoPE + paged KV append into exclusively owned pages.
 * ("FlashInfer parity matrix": rows Standard RoPE and Fused RoPE plus paged
 * append; section "Paged KV ownership difference": append accepts an
 * authoritative per-page reference-count snapshot and writes only pages whose
 * count is one.  "Oxide Infer" README, "Operator surface": BF16 NeoX RoPE with
 * explicit positions.)
 *
 * For every token t (0 <= t < nnz) of sequence b = batch_indices[t] at
 * position p = positions[t] (one int32 serves as the RoPE position and the
 * token's logical KV slot):
 *   - k_rot = RoPE(k_in[t], p), v = v_in[t]   ([num_kv_heads][128] each)
 *   - both are stored at slot p % 16 of page page_indices[page_indptr[b] + p/16]
 *   - if q_in != NULL: q_out[t] = RoPE(q_in[t], p)   ([num_qo_heads][128])
 * RoPE: pair (i, i + 64), angle a = p * rope_theta^(-2i/128) (evaluated in
 * double precision), (x_i cos a - x_{i+64} sin a, x_{i+64} cos a + x_i sin a),
 * rounded once to bf16.
 *
 * All or nothing: a check pass validates every token (batch index in
 * [0, batch), position in [0, 16 * pages listed for b), page id in
 * [0, num_pages), page_refcounts[page] == 1) and records, per work-group, the
 * smallest failing token in the workspace; the writing kernel reduces those
 * records first and writes only if no token failed.  status[0] = 0 or the
 * OXA_DEV_* code of the lowest failing token, status[1] = that token or -1.
 * On failure no pool byte and no q_out byte changes.  Two tokens naming the
 * same (page, slot) break the contract (the result is unspecified).
 *
 * Shapes: q_in/q_out [nnz][num_qo_heads][128]; k_in/v_in [nnz][num_kv_heads][128];
 * batch_indices/positions [nnz]; page_indptr [batch+1];
 * page_indices [num_page_entries]; page_refcounts [num_pages]; status [2].
 * q_out may equal q_in (in place) but may not overlap it otherwise; q_in and
 * q_out are both NULL or both non-NULL (num_qo_heads is then ignored).
 * workspace: device scratch of oxa_paged_append_rope_workspace_bytes(nnz)
 * bytes (16-byte aligned, any contents), used for the call only.
 * Ranges: 0 <= nnz (0 = no-op apart from status; the per-token pointers
 * q_in, q_out, k_in, v_in, batch_indices, positions may then be NULL),
 * 1 <= batch.
 */
oxa_status oxa_paged_append_rope(
    hipStream_t stream,
    const uint16_t* q_in, uint16_t* q_out, int32_t num_qo_heads,
    const uint16_t* k_in, const uint16_t* v_in, int32_t num_kv_heads, int32_t head_dim,
    const int32_t* batch_indices, const int32_t* positions, int32_t nnz,
    uint16_t* k_pages, uint16_t* v_pages, int32_t num_pages, int32_t page_size, int32_t layout,
    const int32_t* page_indptr, int32_t batch,
    const int32_t* page_indices, int32_t num_page_entries,
    const int32_t* page_refcounts, float rope_theta,
    void* workspace, size_t workspace_bytes,
    int32_t* status);

/* Workspace bytes oxa_paged_append_rope needs (8192, whatever nnz is). */
size_t oxa_paged_append_rope_workspace_bytes(int32_t nnz);

/*
 * Plain paged KV append into exclusively owned pages: k_in[t] and v_in[t] are
 * stored as they are (no rotation) at slot p % 16 of page
 * page_indices[page_indptr[b] + p / 16], b = batch_indices[t],
 * p = positions[t].  ("Oxide Infer" README, "Operator surface": the KV-cache
 * family lists paged append beside RoPE plus paged append; "FlashInfer parity
 * matrix", "Domain coverage": paged KV append, the standard append; "Paged KV
 * ownership difference": writes only pages whose reference count is one.)
 *
 * Checks, all-or-nothing behaviour, status[2], workspace, layouts, shapes and
 * ranges are those of oxa_paged_append_rope without q and without RoPE.
 */
oxa_status oxa_paged_append(
    hipStream_t stream,
    const uint16_t* k_in, const uint16_t* v_in, int32_t num_kv_heads, int32_t head_dim,
    const int32_t* batch_indices, const int32_t* positions, int32_t nnz,
    uint16_t* k_pages, uint16_t* v_pages, int32_t num_pages, int32_t page_size, int32_t layout,
    const int32_t* page_indptr, int32_t batch,
    const int32_t* page_indices, int32_t num_page_entries,
    const int32_t* page_refcounts,
    void* workspace, size_t workspace_bytes,
    int32_t* status);

/* Workspace bytes oxa_paged_append needs (as oxa_paged_append_rope). */
size_t oxa_paged_append_workspace_bytes(int32_t nnz);

/*
 * Paged batch decode: one query token per sequence over its paged KV.
 * ("FlashInfer parity matrix", Admitted attention matrix: Paged batch decode
 * - MHA, MQA, GQA, mixed lengths, page order, read-only page reuse; Single
 * decode split-K - explicit partitions, F32 partial workspace and a merge.)
 *
 * o[b][h] = sum_j softmax_j(sm_scale * <q[b][h], k_j>) v_j over the
 * seq_lens[b] tokens of sequence b, kv head h / (Hq / Hkv).
 *
 * num_partitions P >= 1 splits each sequence into explicit partitions of
 * C = ceil(ceil(max_seq_len / 16) / P) pages: partition p holds the tokens
 * [16*C*p, min(16*C*(p+1), seq_len)).  With P == 1 one kernel writes o (and
 * lse) directly and no workspace is needed.  With P > 1 the partial states go
 * to the workspace and a merge kernel combines them; the workspace then holds,
 * on completion,
 *     o_part   f32 [batch][num_qo_heads][P][128]  normalised partial outputs
 *     lse_part f32 [batch][num_qo_heads][P]       natural-log partial lse
 *                                                  (-inf for an empty partition,
 *                                                  whose o_part row is 0)
 * laid out back to back from the workspace pointer (o_part first).
 *
 * status (may be NULL) [batch]: status[b] = 0 or the first failing check of
 * sequence b in the order OXA_DEV_SEQ_LEN (1 <= seq_len <= max_seq_len),
 * OXA_DEV_INDPTR (0 <= page_indptr[b] <= page_indptr[b+1] <= num_page_entries
 * and 16 * pages >= seq_len), OXA_DEV_PAGE_RANGE (a needed page id outside
 * [0, num_pages)).  Every status word is written on every call.
 *
 * Shapes: q, o [batch][num_qo_heads][128]; lse [batch][num_qo_heads] or NULL;
 * page_indptr [batch+1]; seq_lens [batch].  Ranges: 1 <= batch,
 * 1 <= max_seq_len, 1 <= num_partitions <= 1024.
 */
oxa_status oxa_paged_decode(
    hipStream_t stream,
    const uint16_t* q, int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
    const uint16_t* k_pages, const uint16_t* v_pages, int32_t num_pages, int32_t page_size,
    int32_t layout,
    const int32_t* page_indptr, const int32_t* page_indices, int32_t num_page_entries,
    const int32_t* seq_lens, int32_t max_seq_len,
    float sm_scale, int32_t num_partitions,
    void* workspace, size_t workspace_bytes,
    uint16_t* o, float* lse, int32_t* status);

/*
 * Allocation-free paged decode, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): oxa_paged_decode with the same arguments, results and
 * status, minus the workspace.  The split-K partial states go to a static
 * scratch array inside the library instead, OXA_DECODE_SCRATCH_BYTES per GPU,
 * which each GPU the library runs on holds until the process ends.  A call
 * whose states need more (oxa_paged_decode_workspace_bytes > the limit, i.e.
 * batch * num_qo_heads * num_partitions > 16256) returns
 * OXA_ERR_SCRATCH_LIMIT and enqueues nothing.  The call allocates and frees
 * nothing; its first call on a device resolves that device's scratch address
 * once.  Every call on one GPU shares that GPU's scratch, so calls that may
 * overlap in time on one GPU (other streams, other host threads) race and
 * must be ordered by the caller.  After a split call the scratch holds the
 * partial states laid out as oxa_paged_decode's workspace.
 */
#define OXA_DECODE_SCRATCH_BYTES ((size_t)8 << 20)
oxa_status oxa_paged_decode_noalloc(
    hipStream_t stream,
    const uint16_t* q, int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
    const uint16_t* k_pages, const uint16_t* v_pages, int32_t num_pages, int32_t page_size,
    int32_t layout,
    const int32_t* page_indptr, const int32_t* page_indices, int32_t num_page_entries,
    const int32_t* seq_lens, int32_t max_seq_len,
    float sm_scale, int32_t num_partitions,
    uint16_t* o, float* lse, int32_t* status);

/* Workspace bytes oxa_paged_decode needs (0 for num_partitions == 1). */
size_t oxa_paged_decode_workspace_bytes(int32_t batch, int32_t num_qo_heads, int32_t head_dim,
                                        int32_t num_partitions);

/*
 * Workspace bytes of oxa_paged_decode's load-balanced mode (0 when the shape
 * has no such mode: batch * num_partitions > 2048).  A workspace of at least
 * this size makes oxa_paged_decode cut the pages of all sequences (or of
 * their partitions), laid end to end, into equal ranges, one per compute
 * unit, and merge the pieces of the units a range boundary cuts in a second
 * kernel, so a batch of mixed lengths takes the time of its total rather than
 * of its longest sequence.  The results are those of the direct mode (the
 * same attention, summed in another order), and with P > 1 the workspace
 * starts with the same partition states; the rest of it is scratch.  Small
 * calls (fewer than 64 pages of the largest possible total) take the direct
 * mode whatever the workspace.
 */
size_t oxa_paged_decode_balanced_workspace_bytes(int32_t batch, int32_t num_qo_heads,
                                                 int32_t head_dim, int32_t num_partitions);

/*
 * Ragged prefill: sequence b's query rows q[qo_indptr[b] .. qo_indptr[b+1])
 * attend to k/v[kv_indptr[b] .. kv_indptr[b+1]).  ("FlashInfer parity
 * matrix", Admitted attention matrix: Ragged causal prefill.)
 *
 * causal != 0 masks bottom-right: query row i of a sequence with qo_len rows
 * and kv_len keys sees keys j <= i + (kv_len - qo_len).  causal == 0 lets every
 * row see every key.
 *
 * status (may be NULL) [batch]: 0 or the first failing check of sequence b:
 * OXA_DEV_INDPTR (each indptr non-decreasing from >= 0 and within nnz),
 * OXA_DEV_SEQ_LEN (qo_len <= max_qo_len, kv_len <= max_kv_len, kv_len >= 1
 * when qo_len >= 1), OXA_DEV_CAUSAL (causal and qo_len > kv_len).
 *
 * Shapes: q, o [nnz_qo][num_qo_heads][128]; k, v [nnz_kv][num_kv_heads][128];
 * lse [nnz_qo][num_qo_heads] or NULL; qo_indptr, kv_indptr [batch+1].
 *
 * Workspace (optional; NULL disables what follows): a call too small to fill
 * the GPU - at most nnz_qo * num_qo_heads = 32768 query rows times heads, and
 * few enough (query tile, kv head) items to leave at least half of the compute
 * units idle - may cut each item's keys into up to 8 chunks that run in
 * parallel, and merge their states as the split-K decode does (same
 * attention up to f32 rounding order).  That needs a workspace of
 * oxa_ragged_prefill_workspace_bytes(...) bytes (16-byte aligned, any
 * contents, used for the call only; the query returns 0 for calls too large
 * to split, whose workspace is then unused).  With the split, rows of o
 * outside every valid sequence are unspecified.
 * Ranges: 1 <= batch, 0 <= nnz_qo, nnz_kv; 1 <= max_kv_len;
 * 1 <= max_qo_len <= 4096 * BM, where BM = 256 / min(Hq / Hkv, 256) query
 * rows form one tile (for example 262144 rows for four q heads per kv head).
 */
oxa_status oxa_ragged_prefill(
    hipStream_t stream,
    const uint16_t* q, const uint16_t* k, const uint16_t* v,
    const int32_t* qo_indptr, const int32_t* kv_indptr,
    int32_t batch, int32_t nnz_qo, int32_t nnz_kv,
    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_qo_len, int32_t max_kv_len, int32_t causal, float sm_scale,
    void* workspace, size_t workspace_bytes,
    uint16_t* o, float* lse, int32_t* status);

/* Workspace bytes that let oxa_ragged_prefill split small calls' keys (0 when
 * nnz_qo * num_qo_heads exceeds 32768 or the arguments are invalid). */
size_t oxa_ragged_prefill_workspace_bytes(int32_t batch, int32_t nnz_qo, int32_t num_qo_heads,
                                          int32_t head_dim);

/*
 * Paged prefill: sequence b's query rows q[qo_indptr[b] .. qo_indptr[b+1])
 * attend to the first seq_lens[b] tokens of its paged KV.  ("FlashInfer
 * parity matrix", Admitted attention matrix: Paged causal prefill; Graph
 * evidence: invalid-page rejection.)  Causal alignment as in
 * oxa_ragged_prefill with kv_len = seq_lens[b].
 *
 * status (may be NULL) [batch]: 0 or the first failing check of sequence b:
 * OXA_DEV_INDPTR (qo_indptr / page_indptr ranges), OXA_DEV_SEQ_LEN
 * (qo_len <= max_qo_len, 0 <= seq_len <= max_seq_len, seq_len >= 1 when
 * qo_len >= 1), OXA_DEV_INDPTR (too few pages for seq_len), OXA_DEV_CAUSAL,
 * OXA_DEV_PAGE_RANGE.
 *
 * Shapes: q, o [nnz_qo][num_qo_heads][128]; lse [nnz_qo][num_qo_heads] or
 * NULL; qo_indptr, page_indptr [batch+1]; seq_lens [batch].
 * Workspace as for oxa_ragged_prefill (size: oxa_paged_prefill_workspace_bytes).
 * Ranges as for oxa_ragged_prefill, with max_seq_len in place of max_kv_len.
 */
oxa_status oxa_paged_prefill(
    hipStream_t stream,
    const uint16_t* q, const int32_t* qo_indptr,
    const uint16_t* k_pages, const uint16_t* v_pages, int32_t num_pages, int32_t page_size,
    int32_t layout,
    const int32_t* page_indptr, const int32_t* page_indices, int32_t num_page_entries,
    const int32_t* seq_lens,
    int32_t batch, int32_t nnz_qo, int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_qo_len, int32_t max_seq_len, int32_t causal, float sm_scale,
    void* workspace, size_t workspace_bytes,
    uint16_t* o, float* lse, int32_t* status);

/* As oxa_ragged_prefill_workspace_bytes, for oxa_paged_prefill. */
size_t oxa_paged_prefill_workspace_bytes(int32_t batch, int32_t nnz_qo, int32_t num_qo_heads,
                                         int32_t head_dim);

/*
 * Attention-state merge.  ("FlashInfer parity matrix": section Domain
 * coverage, Attention state and cascade - the state merge; the merge of the
 * Single decode split-K row of the Admitted attention matrix.)
 *
 * The state of one (row, head) over a set of keys is the softmax attention
 * output v over that set ([128] values) and lse, the natural-log
 * log-sum-exp of its scaled scores (f32).  States of disjoint key sets
 * combine into the state of their union:
 *     lse = ln sum_s exp(lse_s),     v = sum_s exp(lse_s - lse) * v_s
 * in f32.  A state with lse_s = -inf (no keys) contributes nothing, whatever
 * its v holds; if every state is empty, v = 0 and lse = -inf.  lse values
 * must be finite or -inf (otherwise the result is unspecified).
 *
 * v_dtype is the type of the input states, out_dtype that of v_out
 * (OXA_DTYPE_BF16 as uint16 bits, rounded to nearest even on output, or
 * OXA_DTYPE_F32); lse_out (may be NULL) is f32.
 *
 * oxa_merge_states: S states per (row, head), stored row-major:
 *   v   [num_rows][num_states][num_heads][128]   v_dtype
 *   lse [num_rows][num_states][num_heads]        f32
 *   v_out [num_rows][num_heads][128] out_dtype,  lse_out [num_rows][num_heads]
 * Outputs may not overlap inputs.
 *
 * oxa_merge_state_pair: two states per (row, head) in separate tensors
 *   v_a, v_b [num_rows][num_heads][128] v_dtype;  lse_a, lse_b [num_rows][num_heads]
 *   v_out [num_rows][num_heads][128] out_dtype,   lse_out [num_rows][num_heads]
 * In place: v_out may be exactly v_a or v_b (when out_dtype == v_dtype) and
 * lse_out exactly lse_a or lse_b; any other overlap is rejected.
 *
 * Ranges: 0 <= num_rows (0 = no-op; the pointers may then be NULL),
 * 1 <= num_states, 1 <= num_heads, head_dim == 128.  Alignment: v tensors 16
 * bytes, lse tensors 4.  No workspace, no status: the merge has no
 * data-dependent failure.
 */
oxa_status oxa_merge_states(
    hipStream_t stream,
    const void* v, const float* lse, int32_t v_dtype,
    int32_t num_rows, int32_t num_states, int32_t num_heads, int32_t head_dim,
    void* v_out, int32_t out_dtype, float* lse_out);

oxa_status oxa_merge_state_pair(
    hipStream_t stream,
    const void* v_a, const float* lse_a, const void* v_b, const float* lse_b, int32_t v_dtype,
    int32_t num_rows, int32_t num_heads, int32_t head_dim,
    void* v_out, int32_t out_dtype, float* lse_out);

/*
 * Standalone NeoX RoPE on q and k at explicit positions.  ("FlashInfer parity
 * matrix": Admitted attention matrix, row Standard RoPE - head dim 128, NeoX
 * split-half, explicit int32 positions; Domain coverage, RoPE - the standard
 * and Llama 3.1 variants.  "Oxide Infer" README, Operator surface: BF16 NeoX
 * RoPE with explicit positions.)
 *
 * For every token t < nnz at position p = positions[t] (any int32; negative
 * positions rotate backwards) and every head row x of q[t] and k[t]: pair
 * (x_i, x_{i+64}), i < 64, becomes (x_i cos a - x_{i+64} sin a,
 * x_{i+64} cos a + x_i sin a) with a = p * f_i, evaluated in double precision
 * and rounded once to bf16 (nearest even) - the same rotation the fused
 * oxa_paged_append_rope applies.
 *
 * oxa_rope_neox:    f_i = rope_theta^(-2i/128).
 * oxa_rope_llama31: the Llama 3.1 rescaling of that table.  With wavelength
 *   w_i = 2 pi / f_i, L = original_max_position: f_i stays if
 *   w_i < L / high_freq_factor, becomes f_i / factor if w_i > L / low_freq_factor,
 *   and in between (1 - m) f_i / factor + m f_i with
 *   m = (L / w_i - low_freq_factor) / (high_freq_factor - low_freq_factor).
 *   Requires factor > 0, 0 < low_freq_factor < high_freq_factor, L >= 1.
 *
 * Shapes: q_in, q_out [nnz][num_qo_heads][128]; k_in, k_out
 * [nnz][num_kv_heads][128]; positions [nnz].  q_in and q_out are both NULL
 * (q is skipped; num_qo_heads is ignored) or both set, likewise k_in / k_out;
 * at least one of the two is set.  q_out may equal q_in and k_out k_in (in
 * place); any other overlap between the regions is rejected.  nnz == 0 is a
 * no-op (the tensor pointers may then be NULL).  rope_theta must be finite
 * and > 0.  No workspace, no status: nothing here depends on the data.
 */
oxa_status oxa_rope_neox(
    hipStream_t stream,
    const uint16_t* q_in, uint16_t* q_out, int32_t num_qo_heads,
    const uint16_t* k_in, uint16_t* k_out, int32_t num_kv_heads, int32_t head_dim,
    const int32_t* positions, int32_t nnz, float rope_theta);

oxa_status oxa_rope_llama31(
    hipStream_t stream,
    const uint16_t* q_in, uint16_t* q_out, int32_t num_qo_heads,
    const uint16_t* k_in, uint16_t* k_out, int32_t num_kv_heads, int32_t head_dim,
    const int32_t* positions, int32_t nnz, float rope_theta,
    float factor, float low_freq_factor, float high_freq_factor,
    int32_t original_max_position);

#ifdef __cplusplus
}
#endif

#endif /* OXA_H */
