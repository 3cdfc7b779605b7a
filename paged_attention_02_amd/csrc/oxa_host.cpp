// C-ABI entry points of liboxa: argument validation, workspace sizing and
// launch of the gfx950 kernels.
//
// Runtime rules from the "Oxide Infer" README (sections "One execution model"
// and "Providers"): the caller selects the stream; read and write regions are
// typed and checked for span, alignment, aliasing and capacity before anything
// is enqueued; workspace requirements are explicit; device-detected failures
// are typed status codes; enqueue neither tunes nor falls back silently.
// Every check below runs on the host before the first HIP call, so a rejected
// call touches no device state.
#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "../../include/oxa.h"
#include "kernels.h"

namespace {

struct Region {
  const void* ptr;
  uint64_t bytes;
};

bool overlaps(const Region& a, const Region& b) {
  if (a.ptr == nullptr || b.ptr == nullptr || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.ptr), b0 = reinterpret_cast<uintptr_t>(b.ptr);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

bool aligned(const void* p, uintptr_t a) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Outputs must not overlap any input or one another.
bool any_alias(const Region* outs, int nout, const Region* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlaps(outs[i], ins[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlaps(outs[i], outs[j])) return true;
  }
  return false;
}

constexpr uint64_t kRowBytes = OXA_HEAD_DIM * 2;  // one bf16 head row
static_assert(OXA_DECODE_SCRATCH_BYTES == oxa::kDecodeScratchBytes,
              "the header states the static decode scratch size");
constexpr int kMaxGridYZ = 65535;
constexpr uint64_t kMaxPrefillTiles = 4096;

oxa_status check_heads(int32_t hq, int32_t hkv, int32_t head_dim) {
  if (head_dim != OXA_HEAD_DIM) return OXA_ERR_UNSUPPORTED;
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return OXA_ERR_SHAPE;
  return OXA_OK;
}

oxa_status check_paging(int32_t page_size, int32_t layout, int32_t num_pages,
                        int32_t num_page_entries) {
  if (page_size != OXA_PAGE_SIZE) return OXA_ERR_UNSUPPORTED;
  if (layout != OXA_LAYOUT_NHD && layout != OXA_LAYOUT_HND) return OXA_ERR_UNSUPPORTED;
  if (num_pages < 1 || num_page_entries < 0) return OXA_ERR_SHAPE;
  return OXA_OK;
}

oxa_status launch_status(hipError_t e) { return e == hipSuccess ? OXA_OK : OXA_ERR_LAUNCH; }

bool dtype_ok(int32_t t) { return t == OXA_DTYPE_BF16 || t == OXA_DTYPE_F32; }
uint64_t dtype_bytes(int32_t t) { return t == OXA_DTYPE_F32 ? 4 : 2; }

// The merge kernels use one work-group per few (row, head) units.
oxa_status check_merge_shape(int32_t num_rows, int32_t num_states, int32_t num_heads,
                             int32_t head_dim, int32_t v_dtype, int32_t out_dtype) {
  if (head_dim != OXA_HEAD_DIM || !dtype_ok(v_dtype) || !dtype_ok(out_dtype))
    return OXA_ERR_UNSUPPORTED;
  if (num_rows < 0 || num_states < 1 || num_heads < 1) return OXA_ERR_SHAPE;
  const int64_t units = (int64_t)num_rows * num_heads;
  if (oxa::merge_states_groups(units, v_dtype == OXA_DTYPE_F32) > 0x7fffffffll)
    return OXA_ERR_SHAPE;
  return OXA_OK;
}

// The Llama 3.1 frequency table, evaluated step by step in double precision
// without fused multiply-adds.
void llama31_table(double theta, double factor, double low, double high, int32_t orig,
                   double* out) {
#pragma clang fp contract(off)
  const double low_wl = (double)orig / low;
  const double high_wl = (double)orig / high;
  for (int i = 0; i < 64; ++i) {
    const double base = std::pow(theta, -2.0 * (double)i / (double)OXA_HEAD_DIM);
    const double wl = 2.0 * M_PI / base;
    const double smooth = ((double)orig / wl - low) / (high - low);
    const double blended = (1.0 - smooth) * base / factor + smooth * base;
    double f = wl > low_wl ? base / factor : blended;
    if (wl < high_wl) f = base;
    out[i] = f;
  }
}


// Query tiles per sequence for the given head grouping (256 columns per
// work-group, BM = 256 / min(group, 256) rows each).  The prefill schedule
// orders at most kMaxPrefillTiles tile indices.
uint64_t prefill_tiles(int32_t hq, int32_t hkv, int32_t max_qo_len) {
  const int32_t group = hq / hkv;
  const int32_t gwg = group < 256 ? group : 256;
  const int32_t bm = 256 / gwg;
  return ((uint64_t)max_qo_len + bm - 1) / bm;
}


// Split-K partition states of a decode call (o_part then lse_part, f32);
// 0 for a call without partitions.
uint64_t decode_state_bytes(int32_t batch, int32_t hq, int32_t partitions) {
  if (partitions <= 1) return 0;
  const uint64_t rows = (uint64_t)batch * hq * partitions;
  return rows * OXA_HEAD_DIM * 4 + rows * 4;
}

uint64_t align256(uint64_t x) { return (x + 255) / 256 * 256; }

// Workspace of the load-balanced decode: the partition states, the unit page
// starts (int32 [units + 1]) and the piece states of at most
// kBalancedMaxRanges + units pieces (o f32 [..][hq][128], then lse f32 [..][hq]).
uint64_t decode_balanced_bytes(int32_t batch, int32_t hq, int32_t partitions) {
  const uint64_t units = (uint64_t)batch * partitions;
  const uint64_t slots = (uint64_t)oxa::kBalancedMaxRanges + units;
  return align256(decode_state_bytes(batch, hq, partitions)) + align256((units + 1) * 4) +
         align256(slots * hq * OXA_HEAD_DIM * 4) + slots * hq * 4;
}

// Checks shared by both RoPE entry points; fills everything but the table.
oxa_status rope_setup(const uint16_t* q_in, uint16_t* q_out, int32_t num_qo_heads,
                      const uint16_t* k_in, uint16_t* k_out, int32_t num_kv_heads,
                      int32_t head_dim, const int32_t* positions, int32_t nnz, float rope_theta,
                      oxa::RopeLaunch* a) {
  if ((q_in == nullptr) != (q_out == nullptr) || (k_in == nullptr) != (k_out == nullptr))
    return OXA_ERR_NULL;
  const bool has_q = q_in != nullptr, has_k = k_in != nullptr;
  if (nnz != 0 && ((!has_q && !has_k) || positions == nullptr)) return OXA_ERR_NULL;
  if (head_dim != OXA_HEAD_DIM) return OXA_ERR_UNSUPPORTED;
  if (nnz < 0 || (has_q && num_qo_heads < 1) || (has_k && num_kv_heads < 1)) return OXA_ERR_SHAPE;
  if (!(rope_theta > 0.f) || !std::isfinite(rope_theta)) return OXA_ERR_SHAPE;
  if (!aligned(q_in, 16) || !aligned(q_out, 16) || !aligned(k_in, 16) || !aligned(k_out, 16) ||
      !aligned(positions, 4))
    return OXA_ERR_ALIGN;
  const uint64_t n = (uint64_t)nnz;
  const uint64_t qb = has_q ? n * (uint64_t)num_qo_heads * kRowBytes : 0;
  const uint64_t kb = has_k ? n * (uint64_t)num_kv_heads * kRowBytes : 0;
  const Region qi{q_in, qb}, ki{k_in, kb}, pi{positions, n * 4};
  const Region qo{q_out == q_in ? nullptr : q_out, qb}, ko{k_out == k_in ? nullptr : k_out, kb};
  // outputs written in place count as their input region
  const Region qw{q_out, qb}, kw{k_out, kb};
  if (overlaps(qw, kw) || overlaps(qw, ki) || overlaps(qw, pi) || overlaps(kw, qi) ||
      overlaps(kw, pi) || overlaps(qo, qi) || overlaps(ko, ki))
    return OXA_ERR_ALIAS;
  a->q_in = q_in;
  a->q_out = q_out;
  a->k_in = k_in;
  a->k_out = k_out;
  a->positions = positions;
  a->hq = has_q ? num_qo_heads : 0;
  a->hkv = has_k ? num_kv_heads : 0;
  a->nnz = nnz;
  return OXA_OK;
}

// Prefill workspace for the key-range split of small calls: the chunk states
// (f32 [kPrefillMaxSplit][nnz_qo][hq][128]) then their lse, 256-byte aligned;
// 0 when the call is too large to split.
uint64_t prefill_split_o_bytes(int32_t nnz_qo, int32_t hq) {
  return ((uint64_t)oxa::kPrefillMaxSplit * nnz_qo * hq * OXA_HEAD_DIM * 4 + 255) / 256 * 256;
}

size_t prefill_split_bytes(int32_t batch, int32_t nnz_qo, int32_t hq, int32_t head_dim) {
  if (batch < 1 || nnz_qo < 1 || hq < 1 || head_dim != OXA_HEAD_DIM ||
      (int64_t)nnz_qo * hq > oxa::kPrefillSplitMaxRowHeads)
    return 0;
  return (size_t)(prefill_split_o_bytes(nnz_qo, hq) +
                  (uint64_t)oxa::kPrefillMaxSplit * nnz_qo * hq * 4);
}

// Workspace checks shared by both prefills; fills the split fields.
oxa_status prefill_workspace(int32_t batch, int32_t nnz_qo, int32_t hq, void* workspace,
                             size_t workspace_bytes, oxa::PrefillLaunch* a, Region* region) {
  a->ws_o = nullptr;
  a->ws_lse = nullptr;
  a->max_split = 1;
  *region = Region{nullptr, 0};
  if (workspace == nullptr) return OXA_OK;
  if (!aligned(workspace, 16)) return OXA_ERR_ALIGN;
  const size_t need = prefill_split_bytes(batch, nnz_qo, hq, OXA_HEAD_DIM);
  if (need == 0) return OXA_OK;  // too large to split: the workspace is not used
  if (workspace_bytes < need) return OXA_ERR_WORKSPACE;
  unsigned char* w = static_cast<unsigned char*>(workspace);
  a->ws_o = reinterpret_cast<float*>(w);
  a->ws_lse = reinterpret_cast<float*>(w + prefill_split_o_bytes(nnz_qo, hq));
  a->max_split = oxa::kPrefillMaxSplit;
  *region = Region{workspace, need};
  return OXA_OK;
}

// Both paged appends: validation, then the check pass and the writer.
oxa_status paged_append_impl(hipStream_t stream, const uint16_t* q_in, uint16_t* q_out,
                             int32_t num_qo_heads, const uint16_t* k_in,
                             const uint16_t* v_in, int32_t num_kv_heads, int32_t head_dim,
                             const int32_t* batch_indices, const int32_t* positions,
                             int32_t nnz, uint16_t* k_pages, uint16_t* v_pages,
                             int32_t num_pages, int32_t page_size, int32_t layout,
                             const int32_t* page_indptr, int32_t batch,
                             const int32_t* page_indices, int32_t num_page_entries,
                             const int32_t* page_refcounts, bool rope, float rope_theta,
                             void* workspace, size_t workspace_bytes, int32_t* status) {
  // with no tokens the per-token arrays may be absent (empty tensors)
  if ((nnz != 0 && (!k_in || !v_in || !batch_indices || !positions)) || !k_pages || !v_pages ||
      !page_indptr || !page_indices || !page_refcounts || !status)
    return OXA_ERR_NULL;
  if ((q_in == nullptr) != (q_out == nullptr)) return OXA_ERR_NULL;
  const bool has_q = q_in != nullptr;
  if (head_dim != OXA_HEAD_DIM) return OXA_ERR_UNSUPPORTED;
  if (num_kv_heads < 1 || (has_q && num_qo_heads < 1)) return OXA_ERR_SHAPE;
  if (oxa_status s = check_paging(page_size, layout, num_pages, num_page_entries)) return s;
  if (nnz < 0 || batch < 1) return OXA_ERR_SHAPE;
  if (rope && (!(rope_theta > 0.f) || !std::isfinite(rope_theta))) return OXA_ERR_SHAPE;
  if (!aligned(q_in, 16) || !aligned(q_out, 16) || !aligned(k_in, 16) || !aligned(v_in, 16) ||
      !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(batch_indices, 4) ||
      !aligned(positions, 4) || !aligned(page_indptr, 4) || !aligned(page_indices, 4) ||
      !aligned(page_refcounts, 4) || !aligned(status, 4) || !aligned(workspace, 16))
    return OXA_ERR_ALIGN;
  const size_t need = (size_t)oxa::kAppendCheckGroups * 8;
  if (workspace == nullptr || workspace_bytes < need) return OXA_ERR_WORKSPACE;

  const uint64_t n = (uint64_t)nnz;
  const uint64_t qbytes = has_q ? n * (uint64_t)num_qo_heads * kRowBytes : 0;
  const uint64_t pool = (uint64_t)num_pages * OXA_PAGE_SIZE * (uint64_t)num_kv_heads * kRowBytes;
  const Region ins[] = {{q_in, qbytes},
                        {k_in, n * num_kv_heads * kRowBytes},
                        {v_in, n * num_kv_heads * kRowBytes},
                        {batch_indices, n * 4},
                        {positions, n * 4},
                        {page_indptr, ((uint64_t)batch + 1) * 4},
                        {page_indices, (uint64_t)num_page_entries * 4},
                        {page_refcounts, (uint64_t)num_pages * 4}};
  // q_out == q_in (exactly) is the in-place form; any other overlap is rejected
  const bool in_place = has_q && q_out == q_in;
  const Region outs[] = {{k_pages, pool}, {v_pages, pool}, {status, 8},
                         {workspace, need}, {in_place ? nullptr : q_out, qbytes}};
  if (any_alias(outs, 5, ins, 8)) return OXA_ERR_ALIAS;
  if (in_place) {
    const Region qr{q_in, qbytes};
    for (int i = 1; i < 8; ++i)
      if (overlaps(qr, ins[i])) return OXA_ERR_ALIAS;
    for (int i = 0; i < 4; ++i)
      if (overlaps(qr, outs[i])) return OXA_ERR_ALIAS;
  }

  oxa::AppendLaunch a;
  a.q_in = q_in;
  a.q_out = q_out;
  a.k_in = k_in;
  a.v_in = v_in;
  a.batch_indices = batch_indices;
  a.positions = positions;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.page_indptr = page_indptr;
  a.page_indices = page_indices;
  a.page_refcounts = page_refcounts;
  a.status = status;
  a.check = static_cast<int32_t*>(workspace);
  a.hq = has_q ? num_qo_heads : 0;
  a.hkv = num_kv_heads;
  a.nnz = nnz;
  a.num_pages = num_pages;
  a.layout = layout;
  a.batch = batch;
  a.num_page_entries = num_page_entries;
  a.rope = rope ? 1 : 0;
  for (int i = 0; i < 64; ++i)
    a.inv_freq[i] =
        rope ? std::pow((double)rope_theta, -2.0 * (double)i / (double)OXA_HEAD_DIM) : 0.0;
  return launch_status(oxa::launch_paged_append_rope(a, stream));
}

}  // namespace

extern "C" {

int32_t oxa_abi_version(void) { return OXA_ABI_VERSION; }

const char* oxa_status_string(int32_t code) {
  switch (code) {
    case OXA_OK: return "OXA_OK";
    case OXA_ERR_NULL: return "OXA_ERR_NULL";
    case OXA_ERR_UNSUPPORTED: return "OXA_ERR_UNSUPPORTED";
    case OXA_ERR_SHAPE: return "OXA_ERR_SHAPE";
    case OXA_ERR_ALIGN: return "OXA_ERR_ALIGN";
    case OXA_ERR_ALIAS: return "OXA_ERR_ALIAS";
    case OXA_ERR_WORKSPACE: return "OXA_ERR_WORKSPACE";
    case OXA_ERR_LAUNCH: return "OXA_ERR_LAUNCH";
    case OXA_ERR_SCRATCH_LIMIT: return "OXA_ERR_SCRATCH_LIMIT";
    case OXA_DEV_PAGE_RANGE: return "OXA_DEV_PAGE_RANGE";
    case OXA_DEV_INDPTR: return "OXA_DEV_INDPTR";
    case OXA_DEV_SEQ_LEN: return "OXA_DEV_SEQ_LEN";
    case OXA_DEV_CAUSAL: return "OXA_DEV_CAUSAL";
    case OXA_DEV_NOT_EXCLUSIVE: return "OXA_DEV_NOT_EXCLUSIVE";
    case OXA_DEV_CAPACITY: return "OXA_DEV_CAPACITY";
    case OXA_DEV_BATCH_INDEX: return "OXA_DEV_BATCH_INDEX";
    default: return "unknown";
  }
}

// ---------------------------------------------------------------- append

size_t oxa_paged_append_rope_workspace_bytes(int32_t nnz) {
  (void)nnz;  // one record per check work-group, whatever the token count
  return (size_t)oxa::kAppendCheckGroups * 8;
}

oxa_status oxa_paged_append_rope(hipStream_t stream, const uint16_t* q_in, uint16_t* q_out,
                                 int32_t num_qo_heads, const uint16_t* k_in,
                                 const uint16_t* v_in, int32_t num_kv_heads, int32_t head_dim,
                                 const int32_t* batch_indices, const int32_t* positions,
                                 int32_t nnz, uint16_t* k_pages, uint16_t* v_pages,
                                 int32_t num_pages, int32_t page_size, int32_t layout,
                                 const int32_t* page_indptr, int32_t batch,
                                 const int32_t* page_indices, int32_t num_page_entries,
                                 const int32_t* page_refcounts, float rope_theta,
                                 void* workspace, size_t workspace_bytes, int32_t* status) {
  return paged_append_impl(stream, q_in, q_out, num_qo_heads, k_in, v_in, num_kv_heads, head_dim,
                           batch_indices, positions, nnz, k_pages, v_pages, num_pages, page_size,
                           layout, page_indptr, batch, page_indices, num_page_entries,
                           page_refcounts, true, rope_theta, workspace, workspace_bytes, status);
}

size_t oxa_paged_append_workspace_bytes(int32_t nnz) {
  return oxa_paged_append_rope_workspace_bytes(nnz);
}

oxa_status oxa_paged_append(hipStream_t stream, const uint16_t* k_in, const uint16_t* v_in,
                            int32_t num_kv_heads, int32_t head_dim, const int32_t* batch_indices,
                            const int32_t* positions, int32_t nnz, uint16_t* k_pages,
                            uint16_t* v_pages, int32_t num_pages, int32_t page_size,
                            int32_t layout, const int32_t* page_indptr, int32_t batch,
                            const int32_t* page_indices, int32_t num_page_entries,
                            const int32_t* page_refcounts, void* workspace,
                            size_t workspace_bytes, int32_t* status) {
  return paged_append_impl(stream, nullptr, nullptr, 0, k_in, v_in, num_kv_heads, head_dim,
                           batch_indices, positions, nnz, k_pages, v_pages, num_pages, page_size,
                           layout, page_indptr, batch, page_indices, num_page_entries,
                           page_refcounts, false, 0.f, workspace, workspace_bytes, status);
}

// ---------------------------------------------------------------- decode

size_t oxa_paged_decode_workspace_bytes(int32_t batch, int32_t num_qo_heads, int32_t head_dim,
                                        int32_t num_partitions) {
  if (batch < 1 || num_qo_heads < 1 || head_dim != OXA_HEAD_DIM || num_partitions < 1 ||
      num_partitions > 1024)
    return 0;
  return (size_t)decode_state_bytes(batch, num_qo_heads, num_partitions);
}

size_t oxa_paged_decode_balanced_workspace_bytes(int32_t batch, int32_t num_qo_heads,
                                                 int32_t head_dim, int32_t num_partitions) {
  if (batch < 1 || num_qo_heads < 1 || head_dim != OXA_HEAD_DIM || num_partitions < 1 ||
      num_partitions > 1024)
    return 0;
  const uint64_t units = (uint64_t)batch * num_partitions;
  if (units > (uint64_t)oxa::kBalancedMaxUnits) return 0;
  return (size_t)decode_balanced_bytes(batch, num_qo_heads, num_partitions);
}

}  // extern "C"

namespace {

// Both decode entry points.  With `use_scratch` the partial states of a split
// call go to the library's per-device static scratch instead of `workspace`.
oxa_status paged_decode_impl(hipStream_t stream, const uint16_t* q, int32_t batch,
                             int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                             const uint16_t* k_pages, const uint16_t* v_pages, int32_t num_pages,
                             int32_t page_size, int32_t layout, const int32_t* page_indptr,
                             const int32_t* page_indices, int32_t num_page_entries,
                             const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                             int32_t num_partitions, void* workspace, size_t workspace_bytes,
                             bool use_scratch, uint16_t* o, float* lse, int32_t* status) {
  if (!q || !k_pages || !v_pages || !page_indptr || !page_indices || !seq_lens || !o)
    return OXA_ERR_NULL;
  if (oxa_status s = check_heads(num_qo_heads, num_kv_heads, head_dim)) return s;
  if (oxa_status s = check_paging(page_size, layout, num_pages, num_page_entries)) return s;
  if (batch < 1 || batch > kMaxGridYZ || max_seq_len < 1 || num_partitions < 1 ||
      num_partitions > 1024 || !(sm_scale >= 0.f) || !std::isfinite(sm_scale))
    return OXA_ERR_SHAPE;
  // one work-group per (sequence, kv head, partition, 16-head tile), padded to 8
  const uint64_t group = (uint64_t)(num_qo_heads / num_kv_heads);
  const uint64_t items = (uint64_t)batch * num_kv_heads * num_partitions;
  if (((items + 7) / 8) * 8 * ((group + 15) / 16) > 0x7fffffffull) return OXA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(o, 16) ||
      !aligned(workspace, 16) || !aligned(lse, 4) || !aligned(status, 4) ||
      !aligned(page_indptr, 4) || !aligned(page_indices, 4) || !aligned(seq_lens, 4))
    return OXA_ERR_ALIGN;
  const size_t need = (size_t)decode_state_bytes(batch, num_qo_heads, num_partitions);
  if (use_scratch) {
    if (need > oxa::kDecodeScratchBytes) return OXA_ERR_SCRATCH_LIMIT;
  } else if (need > 0 && (workspace == nullptr || workspace_bytes < need)) {
    return OXA_ERR_WORKSPACE;
  }
  // The load-balanced path: with a workspace of the full size the query
  // returns, at most kBalancedMaxUnits units, and enough pages for every
  // range to get several (a small call is faster in the direct kernel).
  const uint64_t units = (uint64_t)batch * num_partitions;
  int cus = 0;
  int G = 0;
  size_t used = need;
  if (!use_scratch && workspace != nullptr && units <= (uint64_t)oxa::kBalancedMaxUnits &&
      workspace_bytes >= decode_balanced_bytes(batch, num_qo_heads, num_partitions)) {
    if (oxa::device_cu_count(&cus) != hipSuccess) return OXA_ERR_LAUNCH;
    // one range per compute unit, each of 4 pages or more of the largest
    // possible total (the real total, from seq_lens, is known on the device)
    const uint64_t max_pages = (uint64_t)batch * ((max_seq_len + OXA_PAGE_SIZE - 1) / OXA_PAGE_SIZE);
    const int64_t g = std::min<int64_t>(std::min<int64_t>(oxa::kBalancedMaxRanges, cus),
                                        (int64_t)(max_pages / 4));
    if (max_pages >= 64 && g >= 1) {
      G = (int)g;
      used = (size_t)decode_balanced_bytes(batch, num_qo_heads, num_partitions);
    }
  }

  const uint64_t B = (uint64_t)batch;
  const uint64_t pool = (uint64_t)num_pages * OXA_PAGE_SIZE * (uint64_t)num_kv_heads * kRowBytes;
  const Region ins[] = {{q, B * num_qo_heads * kRowBytes},
                        {k_pages, pool},
                        {v_pages, pool},
                        {page_indptr, (B + 1) * 4},
                        {page_indices, (uint64_t)num_page_entries * 4},
                        {seq_lens, B * 4}};
  const Region outs[] = {{o, B * num_qo_heads * kRowBytes},
                         {lse, lse ? B * num_qo_heads * 4 : 0},
                         {status, status ? B * 4 : 0},
                         {use_scratch ? nullptr : workspace, used}};
  if (any_alias(outs, 4, ins, 6)) return OXA_ERR_ALIAS;
  if (use_scratch && need > 0) {
    // the library's own array: it overlaps nothing the caller owns
    void* p = nullptr;
    if (oxa::decode_scratch_address(&p) != hipSuccess) return OXA_ERR_LAUNCH;
    workspace = p;
  }

  oxa::DecodeLaunch a;
  a.q = q;
  a.k_pages = k_pages;
  a.v_pages = v_pages;
  a.page_indptr = page_indptr;
  a.page_indices = page_indices;
  a.seq_lens = seq_lens;
  a.o = o;
  a.lse = lse;
  a.status = status;
  a.ws_o = need ? static_cast<float*>(workspace) : nullptr;
  a.ws_lse = need ? static_cast<float*>(workspace) + B * num_qo_heads * num_partitions * OXA_HEAD_DIM
                  : nullptr;
  a.batch = batch;
  a.hq = num_qo_heads;
  a.hkv = num_kv_heads;
  a.layout = layout;
  a.num_pages = num_pages;
  a.num_page_entries = num_page_entries;
  a.max_seq_len = max_seq_len;
  a.num_partitions = num_partitions;
  const int32_t max_pages = (max_seq_len + OXA_PAGE_SIZE - 1) / OXA_PAGE_SIZE;
  a.chunk_pages = (max_pages + num_partitions - 1) / num_partitions;
  a.sm_scale = sm_scale;
  if (G > 0) {
    unsigned char* base = static_cast<unsigned char*>(workspace);
    const uint64_t slots = (uint64_t)oxa::kBalancedMaxRanges + units;
    const uint64_t meta_off = align256(need);
    const uint64_t po_off = meta_off + align256((units + 1) * 4);
    const uint64_t pl_off = po_off + align256(slots * num_qo_heads * OXA_HEAD_DIM * 4);
    oxa::BalancedLayout ws;
    ws.meta = reinterpret_cast<int32_t*>(base + meta_off);
    ws.piece_o = reinterpret_cast<float*>(base + po_off);
    ws.piece_lse = reinterpret_cast<float*>(base + pl_off);
    return launch_status(oxa::launch_paged_decode_balanced(a, ws, G, stream));
  }
  return launch_status(oxa::launch_paged_decode(a, stream));
}

}  // namespace

extern "C" {

oxa_status oxa_paged_decode(hipStream_t stream, const uint16_t* q, int32_t batch,
                            int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                            const uint16_t* k_pages, const uint16_t* v_pages, int32_t num_pages,
                            int32_t page_size, int32_t layout, const int32_t* page_indptr,
                            const int32_t* page_indices, int32_t num_page_entries,
                            const int32_t* seq_lens, int32_t max_seq_len, float sm_scale,
                            int32_t num_partitions, void* workspace, size_t workspace_bytes,
                            uint16_t* o, float* lse, int32_t* status) {
  return paged_decode_impl(stream, q, batch, num_qo_heads, num_kv_heads, head_dim, k_pages,
                           v_pages, num_pages, page_size, layout, page_indptr, page_indices,
                           num_page_entries, seq_lens, max_seq_len, sm_scale, num_partitions,
                           workspace, workspace_bytes, false, o, lse, status);
}

oxa_status oxa_paged_decode_noalloc(hipStream_t stream, const uint16_t* q, int32_t batch,
                                    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                                    const uint16_t* k_pages, const uint16_t* v_pages,
                                    int32_t num_pages, int32_t page_size, int32_t layout,
                                    const int32_t* page_indptr, const int32_t* page_indices,
                                    int32_t num_page_entries, const int32_t* seq_lens,
                                    int32_t max_seq_len, float sm_scale, int32_t num_partitions,
                                    uint16_t* o, float* lse, int32_t* status) {
  return paged_decode_impl(stream, q, batch, num_qo_heads, num_kv_heads, head_dim, k_pages,
                           v_pages, num_pages, page_size, layout, page_indptr, page_indices,
                           num_page_entries, seq_lens, max_seq_len, sm_scale, num_partitions,
                           nullptr, 0, true, o, lse, status);
}

// ---------------------------------------------------------------- prefill

size_t oxa_ragged_prefill_workspace_bytes(int32_t batch, int32_t nnz_qo, int32_t num_qo_heads,
                                          int32_t head_dim) {
  return prefill_split_bytes(batch, nnz_qo, num_qo_heads, head_dim);
}
size_t oxa_paged_prefill_workspace_bytes(int32_t batch, int32_t nnz_qo, int32_t num_qo_heads,
                                         int32_t head_dim) {
  return prefill_split_bytes(batch, nnz_qo, num_qo_heads, head_dim);
}


oxa_status oxa_ragged_prefill(hipStream_t stream, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, const int32_t* qo_indptr,
                              const int32_t* kv_indptr, int32_t batch, int32_t nnz_qo,
                              int32_t nnz_kv, int32_t num_qo_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t max_qo_len, int32_t max_kv_len,
                              int32_t causal, float sm_scale, void* workspace,
                              size_t workspace_bytes, uint16_t* o, float* lse, int32_t* status) {
  if (!q || !k || !v || !qo_indptr || !kv_indptr || !o) return OXA_ERR_NULL;
  if (oxa_status s = check_heads(num_qo_heads, num_kv_heads, head_dim)) return s;
  if (batch < 1 || batch > kMaxGridYZ || nnz_qo < 0 || nnz_kv < 0 || max_qo_len < 1 ||
      max_kv_len < 1 || !(sm_scale >= 0.f) || !std::isfinite(sm_scale))
    return OXA_ERR_SHAPE;
  const int32_t group = num_qo_heads / num_kv_heads;
  if (prefill_tiles(num_qo_heads, num_kv_heads, max_qo_len) > kMaxPrefillTiles ||
      (uint64_t)num_kv_heads * (uint64_t)((group + 255) / 256) > 0x7fffffffull)
    return OXA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(status, 4) || !aligned(qo_indptr, 4) || !aligned(kv_indptr, 4))
    return OXA_ERR_ALIGN;
  const uint64_t B = (uint64_t)batch;
  const Region ins[] = {{q, (uint64_t)nnz_qo * num_qo_heads * kRowBytes},
                        {k, (uint64_t)nnz_kv * num_kv_heads * kRowBytes},
                        {v, (uint64_t)nnz_kv * num_kv_heads * kRowBytes},
                        {qo_indptr, (B + 1) * 4},
                        {kv_indptr, (B + 1) * 4}};
  oxa::PrefillLaunch a = {};
  Region ws;
  if (oxa_status st = prefill_workspace(batch, nnz_qo, num_qo_heads, workspace, workspace_bytes,
                                        &a, &ws))
    return st;
  const Region outs[] = {{o, (uint64_t)nnz_qo * num_qo_heads * kRowBytes},
                         {lse, lse ? (uint64_t)nnz_qo * num_qo_heads * 4 : 0},
                         {status, status ? B * 4 : 0},
                         ws};
  if (any_alias(outs, 4, ins, 5)) return OXA_ERR_ALIAS;

  a.q = q;
  a.k = k;
  a.v = v;
  a.qo_indptr = qo_indptr;
  a.kv_indptr = kv_indptr;
  a.o = o;
  a.lse = lse;
  a.status = status;
  a.paged = 0;
  a.layout = 0;
  a.batch = batch;
  a.nnz_qo = nnz_qo;
  a.nnz_kv = nnz_kv;
  a.hq = num_qo_heads;
  a.hkv = num_kv_heads;
  a.max_qo_len = max_qo_len;
  a.max_kv_len = max_kv_len;
  a.causal = causal != 0;
  a.sm_scale = sm_scale;
  return launch_status(oxa::launch_prefill(a, stream));
}

oxa_status oxa_paged_prefill(hipStream_t stream, const uint16_t* q, const int32_t* qo_indptr,
                             const uint16_t* k_pages, const uint16_t* v_pages, int32_t num_pages,
                             int32_t page_size, int32_t layout, const int32_t* page_indptr,
                             const int32_t* page_indices, int32_t num_page_entries,
                             const int32_t* seq_lens, int32_t batch, int32_t nnz_qo,
                             int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_qo_len, int32_t max_seq_len, int32_t causal,
                             float sm_scale, void* workspace, size_t workspace_bytes,
                             uint16_t* o, float* lse, int32_t* status) {
  if (!q || !qo_indptr || !k_pages || !v_pages || !page_indptr || !page_indices || !seq_lens ||
      !o)
    return OXA_ERR_NULL;
  if (oxa_status s = check_heads(num_qo_heads, num_kv_heads, head_dim)) return s;
  if (oxa_status s = check_paging(page_size, layout, num_pages, num_page_entries)) return s;
  if (batch < 1 || batch > kMaxGridYZ || nnz_qo < 0 || max_qo_len < 1 || max_seq_len < 1 ||
      !(sm_scale >= 0.f) || !std::isfinite(sm_scale))
    return OXA_ERR_SHAPE;
  const int32_t group = num_qo_heads / num_kv_heads;
  if (prefill_tiles(num_qo_heads, num_kv_heads, max_qo_len) > kMaxPrefillTiles ||
      (uint64_t)num_kv_heads * (uint64_t)((group + 255) / 256) > 0x7fffffffull)
    return OXA_ERR_SHAPE;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(status, 4) || !aligned(qo_indptr, 4) ||
      !aligned(page_indptr, 4) || !aligned(page_indices, 4) || !aligned(seq_lens, 4))
    return OXA_ERR_ALIGN;
  const uint64_t B = (uint64_t)batch;
  const uint64_t pool = (uint64_t)num_pages * OXA_PAGE_SIZE * (uint64_t)num_kv_heads * kRowBytes;
  const Region ins[] = {{q, (uint64_t)nnz_qo * num_qo_heads * kRowBytes},
                        {k_pages, pool},
                        {v_pages, pool},
                        {qo_indptr, (B + 1) * 4},
                        {page_indptr, (B + 1) * 4},
                        {page_indices, (uint64_t)num_page_entries * 4},
                        {seq_lens, B * 4}};
  oxa::PrefillLaunch a = {};
  Region ws;
  if (oxa_status st = prefill_workspace(batch, nnz_qo, num_qo_heads, workspace, workspace_bytes,
                                        &a, &ws))
    return st;
  const Region outs[] = {{o, (uint64_t)nnz_qo * num_qo_heads * kRowBytes},
                         {lse, lse ? (uint64_t)nnz_qo * num_qo_heads * 4 : 0},
                         {status, status ? B * 4 : 0},
                         ws};
  if (any_alias(outs, 4, ins, 7)) return OXA_ERR_ALIAS;

  a.q = q;
  a.k = k_pages;
  a.v = v_pages;
  a.qo_indptr = qo_indptr;
  a.page_indptr = page_indptr;
  a.page_indices = page_indices;
  a.seq_lens = seq_lens;
  a.o = o;
  a.lse = lse;
  a.status = status;
  a.paged = 1;
  a.layout = layout;
  a.batch = batch;
  a.nnz_qo = nnz_qo;
  a.hq = num_qo_heads;
  a.hkv = num_kv_heads;
  a.max_qo_len = max_qo_len;
  a.max_kv_len = max_seq_len;
  a.causal = causal != 0;
  a.num_pages = num_pages;
  a.num_page_entries = num_page_entries;
  a.sm_scale = sm_scale;
  return launch_status(oxa::launch_prefill(a, stream));
}

// ---------------------------------------------------------------- state merge

oxa_status oxa_merge_states(hipStream_t stream, const void* v, const float* lse, int32_t v_dtype,
                            int32_t num_rows, int32_t num_states, int32_t num_heads,
                            int32_t head_dim, void* v_out, int32_t out_dtype, float* lse_out) {
  if (num_rows != 0 && (!v || !lse || !v_out)) return OXA_ERR_NULL;
  if (oxa_status s = check_merge_shape(num_rows, num_states, num_heads, head_dim, v_dtype,
                                       out_dtype))
    return s;
  if (num_rows == 0) return OXA_OK;
  if (!aligned(v, 16) || !aligned(v_out, 16) || !aligned(lse, 4) || !aligned(lse_out, 4))
    return OXA_ERR_ALIGN;
  const uint64_t units = (uint64_t)num_rows * num_heads;
  const Region ins[] = {{v, units * num_states * OXA_HEAD_DIM * dtype_bytes(v_dtype)},
                        {lse, units * num_states * 4}};
  const Region outs[] = {{v_out, units * OXA_HEAD_DIM * dtype_bytes(out_dtype)},
                         {lse_out, lse_out ? units * 4 : 0}};
  if (any_alias(outs, 2, ins, 2)) return OXA_ERR_ALIAS;

  oxa::MergeLaunch m = {};
  m.v[0] = v;
  m.lse[0] = lse;
  m.v_row = (int64_t)num_states * num_heads * OXA_HEAD_DIM;
  m.v_head = OXA_HEAD_DIM;
  m.v_state = (int64_t)num_heads * OXA_HEAD_DIM;
  m.l_row = (int64_t)num_states * num_heads;
  m.l_head = 1;
  m.l_state = num_heads;
  m.units = (int64_t)units;
  m.heads = num_heads;
  m.states = num_states;
  m.in_f32 = v_dtype == OXA_DTYPE_F32;
  m.out_f32 = out_dtype == OXA_DTYPE_F32;
  m.pair = 0;
  m.out = v_out;
  m.lse_out = lse_out;
  return launch_status(oxa::launch_merge_states(m, stream));
}

oxa_status oxa_merge_state_pair(hipStream_t stream, const void* v_a, const float* lse_a,
                                const void* v_b, const float* lse_b, int32_t v_dtype,
                                int32_t num_rows, int32_t num_heads, int32_t head_dim,
                                void* v_out, int32_t out_dtype, float* lse_out) {
  if (num_rows != 0 && (!v_a || !lse_a || !v_b || !lse_b || !v_out)) return OXA_ERR_NULL;
  if (oxa_status s = check_merge_shape(num_rows, 2, num_heads, head_dim, v_dtype, out_dtype))
    return s;
  if (num_rows == 0) return OXA_OK;
  if (!aligned(v_a, 16) || !aligned(v_b, 16) || !aligned(v_out, 16) || !aligned(lse_a, 4) ||
      !aligned(lse_b, 4) || !aligned(lse_out, 4))
    return OXA_ERR_ALIGN;
  const uint64_t units = (uint64_t)num_rows * num_heads;
  const uint64_t vin = units * OXA_HEAD_DIM * dtype_bytes(v_dtype);
  const uint64_t vout = units * OXA_HEAD_DIM * dtype_bytes(out_dtype);
  // exact aliasing of an output with one input is the in-place form: each
  // (row, head) reads its inputs before it writes the same places
  const bool v_in_place = out_dtype == v_dtype && (v_out == v_a || v_out == v_b);
  const bool l_in_place = lse_out != nullptr && (lse_out == lse_a || lse_out == lse_b);
  const Region vo{v_out, vout};
  const Region lo{lse_out, lse_out ? units * 4 : 0};
  const Region va{v_a, vin}, vb{v_b, vin}, la{lse_a, units * 4}, lb{lse_b, units * 4};
  if (overlaps(vo, lo) || overlaps(vo, la) || overlaps(vo, lb) || overlaps(lo, va) ||
      overlaps(lo, vb))
    return OXA_ERR_ALIAS;
  if (!v_in_place && (overlaps(vo, va) || overlaps(vo, vb))) return OXA_ERR_ALIAS;
  if (!l_in_place && (overlaps(lo, la) || overlaps(lo, lb))) return OXA_ERR_ALIAS;

  oxa::MergeLaunch m = {};
  m.v[0] = v_a;
  m.v[1] = v_b;
  m.lse[0] = lse_a;
  m.lse[1] = lse_b;
  m.v_row = (int64_t)num_heads * OXA_HEAD_DIM;
  m.v_head = OXA_HEAD_DIM;
  m.l_row = num_heads;
  m.l_head = 1;
  m.units = (int64_t)units;
  m.heads = num_heads;
  m.states = 2;
  m.in_f32 = v_dtype == OXA_DTYPE_F32;
  m.out_f32 = out_dtype == OXA_DTYPE_F32;
  m.pair = 1;
  m.out = v_out;
  m.lse_out = lse_out;
  return launch_status(oxa::launch_merge_states(m, stream));
}

// ---------------------------------------------------------------- RoPE


oxa_status oxa_rope_neox(hipStream_t stream, const uint16_t* q_in, uint16_t* q_out,
                         int32_t num_qo_heads, const uint16_t* k_in, uint16_t* k_out,
                         int32_t num_kv_heads, int32_t head_dim, const int32_t* positions,
                         int32_t nnz, float rope_theta) {
  oxa::RopeLaunch a;
  if (oxa_status s = rope_setup(q_in, q_out, num_qo_heads, k_in, k_out, num_kv_heads, head_dim,
                                positions, nnz, rope_theta, &a))
    return s;
  if (nnz == 0) return OXA_OK;
  for (int i = 0; i < 64; ++i)
    a.inv_freq[i] = std::pow((double)rope_theta, -2.0 * (double)i / (double)OXA_HEAD_DIM);
  return launch_status(oxa::launch_rope(a, stream));
}

oxa_status oxa_rope_llama31(hipStream_t stream, const uint16_t* q_in, uint16_t* q_out,
                            int32_t num_qo_heads, const uint16_t* k_in, uint16_t* k_out,
                            int32_t num_kv_heads, int32_t head_dim, const int32_t* positions,
                            int32_t nnz, float rope_theta, float factor, float low_freq_factor,
                            float high_freq_factor, int32_t original_max_position) {
  oxa::RopeLaunch a;
  if (oxa_status s = rope_setup(q_in, q_out, num_qo_heads, k_in, k_out, num_kv_heads, head_dim,
                                positions, nnz, rope_theta, &a))
    return s;
  if (!(factor > 0.f) || !std::isfinite(factor) || !(low_freq_factor > 0.f) ||
      !(high_freq_factor > low_freq_factor) || !std::isfinite(high_freq_factor) ||
      original_max_position < 1)
    return OXA_ERR_SHAPE;
  if (nnz == 0) return OXA_OK;
  llama31_table((double)rope_theta, factor, low_freq_factor, high_freq_factor,
                original_max_position, a.inv_freq);
  return launch_status(oxa::launch_rope(a, stream));
}

}  // extern "C"
