// Paged KV append into exclusively owned pages, fused with NeoX RoPE of k (and
// q) or plain (gfx950).
//
// Operator contract: "FlashInfer parity matrix", section "Admitted attention
// matrix" (rows Standard RoPE - D128 NeoX split-half with explicit I32
// positions - and Fused RoPE plus paged append - explicit tokens with per-page
// reference counts) and section "Paged KV ownership difference" (append takes
// an authoritative reference-count snapshot and writes only pages whose count
// is one); "Oxide Infer" README, section "Operator surface" (BF16 NeoX RoPE
// with explicit positions; paged append and RoPE plus paged append); "FlashInfer
// parity matrix", section "Domain coverage" (paged KV append: the standard
// append beside the fused RoPE one).
//
// Two kernels keep the call all-or-nothing without a host round trip:
//  1. the check pass: each work-group validates a share of the tokens and
//     records its smallest failing token in the workspace;
//  2. the writer: every work-group first reduces those records and returns
//     at once if any token failed; work-group 0 writes status[0..1].
// Angles are evaluated in double precision (position * inv_freq, then sincos),
// the rotation too, and each result is rounded once to bf16.  Positions reach
// tens of thousands of radians, where a float angle would already be wrong in
// its third decimal.
#include "device_common.h"
#include "kernels.h"

namespace oxa {
namespace {

constexpr int kStatusPageRange = 16;
constexpr int kStatusNotExclusive = 20;
constexpr int kStatusCapacity = 21;
constexpr int kStatusBatchIndex = 22;

struct AppendParams {
  const uint16_t* q_in;
  uint16_t* q_out;
  const uint16_t* k_in;
  const uint16_t* v_in;
  const int32_t* batch_indices;
  const int32_t* positions;
  uint16_t* kp;
  uint16_t* vp;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* page_refcounts;
  int32_t* status;
  int32_t* check;  // [check_groups][2]: smallest failing token, its code
  int32_t check_groups;
  int32_t hq, hkv, nnz, num_pages, layout, batch, num_page_entries;
  double inv_freq[64];
};

constexpr int kNone = 0x7fffffff;        // "no failing token"
constexpr int kCheckPer = 4;             // tokens per thread per pass
constexpr int kCheckTile = 256 * kCheckPer;

// Check pass: work-group g checks tokens g*1024 .. g*1024 + 1023 (then every
// gridDim.x*1024 further) and records its smallest failing token and that
// token's code in check[g] (kNone if all pass).  Per pass a thread issues the
// loads of its 4 tokens together, one dependent level at a time (batch index
// and position, then the indptr pair, then the page id, then its refcount),
// through addresses that fall back to a valid dummy word once a token has
// failed, so no load waits behind a branch.
__global__ __launch_bounds__(256) void append_check_kernel(AppendParams p) {
  __shared__ int first_bad, first_code;
  const int tid = threadIdx.x;
  if (tid == 0) first_bad = kNone;
  __syncthreads();
  const int* dummy = p.page_indptr;  // batch >= 1, so at least two words
  int my_t = kNone, my_code = 0;
  for (int base = blockIdx.x * kCheckTile; base < p.nnz && my_t == kNone;
       base += gridDim.x * kCheckTile) {
    // level 1: batch index and position
    int x[kCheckPer], y[kCheckPer], code[kCheckPer];
#pragma unroll
    for (int u = 0; u < kCheckPer; ++u) {
      const int t = base + u * 256 + tid;
      const bool in = t < p.nnz;
      x[u] = *(in ? p.batch_indices + t : dummy);
      y[u] = *(in ? p.positions + t : dummy);
    }
    // level 2: the sequence's page range; x <- page-index slot or -1
    int lo[kCheckPer], hi[kCheckPer];
#pragma unroll
    for (int u = 0; u < kCheckPer; ++u) {
      const bool bok = x[u] >= 0 && x[u] < p.batch;
      lo[u] = *(bok ? p.page_indptr + x[u] : dummy);
      hi[u] = *(bok ? p.page_indptr + x[u] + 1 : dummy);
      code[u] = bok ? 0 : kStatusBatchIndex;
    }
#pragma unroll
    for (int u = 0; u < kCheckPer; ++u) {
      // an indptr that leaves the page-index array gives the sequence no capacity
      const bool ptr_ok = lo[u] >= 0 && hi[u] >= lo[u] && hi[u] <= p.num_page_entries;
      const int64_t cap = ptr_ok ? (int64_t)(hi[u] - lo[u]) * kPage : 0;
      const bool pos_ok = y[u] >= 0 && (int64_t)y[u] < cap;
      if (code[u] == 0 && !pos_ok) code[u] = kStatusCapacity;
      x[u] = code[u] == 0 ? lo[u] + y[u] / kPage : -1;
    }
    // level 3: the page id; x <- page or -1
#pragma unroll
    for (int u = 0; u < kCheckPer; ++u) y[u] = *(x[u] >= 0 ? p.page_indices + x[u] : dummy);
#pragma unroll
    for (int u = 0; u < kCheckPer; ++u) {
      const bool pg_ok = y[u] >= 0 && y[u] < p.num_pages;
      if (code[u] == 0 && !pg_ok) code[u] = kStatusPageRange;
      x[u] = code[u] == 0 ? y[u] : -1;
    }
    // level 4: the page's reference count
#pragma unroll
    for (int u = 0; u < kCheckPer; ++u) y[u] = *(x[u] >= 0 ? p.page_refcounts + x[u] : dummy);
#pragma unroll
    for (int u = 0; u < kCheckPer; ++u) {
      const int t = base + u * 256 + tid;
      if (code[u] == 0 && x[u] >= 0 && y[u] != 1) code[u] = kStatusNotExclusive;
      if (t < p.nnz && code[u] != 0 && my_t == kNone) {
        my_t = t;
        my_code = code[u];
      }
    }
  }
  if (my_t != kNone) atomicMin(&first_bad, my_t);
  __syncthreads();
  if (my_t != kNone && my_t == first_bad) first_code = my_code;  // one thread
  __syncthreads();
  if (tid == 0) {
    p.check[2 * blockIdx.x] = first_bad;
    p.check[2 * blockIdx.x + 1] = first_bad == kNone ? 0 : first_code;
  }
}

// Grid-stride over tokens, one wave per token at a time.  With ROPE, lane l
// evaluates the sin/cos of frequency l and shares it through a wave-private
// LDS slot; lane l then rotates the frequency chunk f = l % 8 (frequencies
// 8f .. 8f+7) of every head it handles.  Without ROPE (the plain append) K is
// copied like V.
template <int LAYOUT, bool ROPE>
__global__ __launch_bounds__(256) void append_rope_kernel(AppendParams p) {
  __shared__ double cs[4][64][2];
  __shared__ int g_bad, g_code;
  // All-or-nothing gate: every work-group reduces the check pass's records;
  // work-group 0 reports the outcome.
  if (threadIdx.x == 0) g_bad = kNone;
  __syncthreads();
  for (int i = threadIdx.x; i < p.check_groups; i += 256) {
    const int tb = p.check[2 * i];
    if (tb != kNone) atomicMin(&g_bad, tb);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < p.check_groups; i += 256)
    if (g_bad != kNone && p.check[2 * i] == g_bad) g_code = p.check[2 * i + 1];
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    p.status[0] = g_bad == kNone ? 0 : g_code;
    p.status[1] = g_bad == kNone ? -1 : g_bad;
  }
  if (g_bad != kNone) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int f = lane & 7;
  const int hsub = lane >> 3;  // 0..7
  const int nwaves = gridDim.x * 4;
  for (int t = blockIdx.x * 4 + wave; t < p.nnz; t += nwaves) {
    // Every token passed the check pass (the gate above), so only its page is
    // looked up here, without branches: the index chain (batch index, indptr,
    // page id) is issued first and waited for only where K and V are stored,
    // after the sin/cos and the q rotation.  The clamps keep every access in
    // bounds whatever the tables hold (a call that reaches this loop has at
    // least one page entry: with none, every token fails the check).
    const int pos = p.positions[t];
    const int b = min(max(p.batch_indices[t], 0), p.batch - 1);
    const int e = min(max(p.page_indptr[b] + (pos >> 4), 0), p.num_page_entries - 1);
    const int page = min(max(p.page_indices[e], 0), p.num_pages - 1);
    const int slot = pos & (kPage - 1);
    const uint16_t* ki = p.k_in + (int64_t)t * p.hkv * kHeadDim;
    const uint16_t* vi = p.v_in + (int64_t)t * p.hkv * kHeadDim;
    if constexpr (!ROPE) {
      // plain append: K and V rows as they are, 16-byte chunks, 16 per head
      for (int cidx = lane; cidx < p.hkv * 16; cidx += 64) {
        const int h = cidx >> 4;
        const int ch = cidx & 15;
        const u32x4_t wk = ldg16(ki + h * kHeadDim + 8 * ch);
        const u32x4_t wv = ldg16(vi + h * kHeadDim + 8 * ch);
        const int64_t row = LAYOUT == 0 ? (((int64_t)page * kPage + slot) * p.hkv + h) * kHeadDim
                                        : (((int64_t)page * p.hkv + h) * kPage + slot) * kHeadDim;
        *reinterpret_cast<u32x4_t*>(p.kp + row + 8 * ch) = wk;
        *reinterpret_cast<u32x4_t*>(p.vp + row + 8 * ch) = wv;
      }
      continue;
    }
    {
      double sl, cl;
      sincos((double)pos * p.inv_freq[lane], &sl, &cl);
      cs[wave][lane][0] = cl;
      cs[wave][lane][1] = sl;
    }
    __builtin_amdgcn_wave_barrier();
    double c[8], s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { c[i] = cs[wave][8 * f + i][0]; s[i] = cs[wave][8 * f + i][1]; }
    __builtin_amdgcn_wave_barrier();

    if (p.q_in != nullptr) {
      const uint16_t* qi = p.q_in + (int64_t)t * p.hq * kHeadDim;
      uint16_t* qo = p.q_out + (int64_t)t * p.hq * kHeadDim;
      for (int h = hsub; h < p.hq; h += 8) {
        const u32x4_t w1 = ldg16(qi + h * kHeadDim + 8 * f);
        const u32x4_t w2 = ldg16(qi + h * kHeadDim + 64 + 8 * f);
        u32x4_t o1, o2;
        rotate_chunk(w1, w2, c, s, &o1, &o2);
        *reinterpret_cast<u32x4_t*>(qo + h * kHeadDim + 8 * f) = o1;
        *reinterpret_cast<u32x4_t*>(qo + h * kHeadDim + 64 + 8 * f) = o2;
      }
    }
    for (int h = hsub; h < p.hkv; h += 8) {
      const u32x4_t w1 = ldg16(ki + h * kHeadDim + 8 * f);
      const u32x4_t w2 = ldg16(ki + h * kHeadDim + 64 + 8 * f);
      u32x4_t o1, o2;
      rotate_chunk(w1, w2, c, s, &o1, &o2);
      const int64_t row = LAYOUT == 0 ? (((int64_t)page * kPage + slot) * p.hkv + h) * kHeadDim
                                      : (((int64_t)page * p.hkv + h) * kPage + slot) * kHeadDim;
      *reinterpret_cast<u32x4_t*>(p.kp + row + 8 * f) = o1;
      *reinterpret_cast<u32x4_t*>(p.kp + row + 64 + 8 * f) = o2;
    }
    // V: copy 16-byte chunks, 16 per head
    for (int cidx = lane; cidx < p.hkv * 16; cidx += 64) {
      const int h = cidx >> 4;
      const int ch = cidx & 15;
      const u32x4_t w = ldg16(vi + h * kHeadDim + 8 * ch);
      const int64_t row = LAYOUT == 0 ? (((int64_t)page * kPage + slot) * p.hkv + h) * kHeadDim
                                      : (((int64_t)page * p.hkv + h) * kPage + slot) * kHeadDim;
      *reinterpret_cast<u32x4_t*>(p.vp + row + 8 * ch) = w;
    }
  }
}

}  // namespace

int append_check_groups(int nnz) {
  int g = (nnz + kCheckTile - 1) / kCheckTile;
  if (g > kAppendCheckGroups) g = kAppendCheckGroups;
  return g < 1 ? 1 : g;
}

hipError_t launch_paged_append_rope(const AppendLaunch& a, hipStream_t stream) {
  AppendParams p;
  p.q_in = a.q_in;
  p.q_out = a.q_out;
  p.k_in = a.k_in;
  p.v_in = a.v_in;
  p.batch_indices = a.batch_indices;
  p.positions = a.positions;
  p.kp = a.k_pages;
  p.vp = a.v_pages;
  p.page_indptr = a.page_indptr;
  p.page_indices = a.page_indices;
  p.page_refcounts = a.page_refcounts;
  p.status = a.status;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.nnz = a.nnz;
  p.num_pages = a.num_pages;
  p.layout = a.layout;
  p.batch = a.batch;
  p.num_page_entries = a.num_page_entries;
  for (int i = 0; i < 64; ++i) p.inv_freq[i] = a.inv_freq[i];
  p.check = a.check;
  p.check_groups = append_check_groups(a.nnz);
  hipError_t e = launch_kernel(append_check_kernel, dim3(p.check_groups), dim3(256), 0, stream, p);
  if (e != hipSuccess) return e;
  // the writer also reports the status, so it runs even for nnz == 0
  int blocks = (a.nnz + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  void (*kernel)(AppendParams) = a.rope ? (a.layout == 0 ? append_rope_kernel<0, true>
                                                           : append_rope_kernel<1, true>)
                                        : (a.layout == 0 ? append_rope_kernel<0, false>
                                                         : append_rope_kernel<1, false>);
  return launch_kernel(kernel, dim3(blocks), dim3(256), 0, stream, p);
}

}  // namespace oxa
