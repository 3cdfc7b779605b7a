// Fused NeoX RoPE + paged KV append into exclusively owned pages (gfx950).
//
// Operator contract: "FlashInfer parity matrix", section "Admitted attention
// matrix" (rows Standard RoPE - D128 NeoX split-half with explicit I32
// positions - and Fused RoPE plus paged append - explicit tokens with per-page
// reference counts) and section "Paged KV ownership difference" (append takes
// an authoritative reference-count snapshot and writes only pages whose count
// is one); "Oxide Infer" README, section "Operator surface" (BF16 NeoX RoPE
// with explicit positions; RoPE plus paged append).
//
// Two kernels keep the call all-or-nothing without a host round trip:
//  1. one work-group checks every token and writes status[0..1];
//  2. the writer kernel returns at once unless status[0] == 0.
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
  int32_t hq, hkv, nnz, num_pages, layout, batch, num_page_entries;
  double inv_freq[64];
};

// Check one token: 0 if it may be written, else its status code.  Also returns
// the target page (valid only when the code is 0).
__device__ __forceinline__ int check_token(const AppendParams& p, int t, int* page_out) {
  const int b = p.batch_indices[t];
  if (b < 0 || b >= p.batch) return kStatusBatchIndex;
  const int lo = p.page_indptr[b];
  const int hi = p.page_indptr[b + 1];
  const int pos = p.positions[t];
  // an indptr that leaves the page-index array gives the sequence no capacity
  const bool ptr_ok = lo >= 0 && hi >= lo && hi <= p.num_page_entries;
  const int64_t cap = ptr_ok ? (int64_t)(hi - lo) * kPage : 0;
  if (pos < 0 || (int64_t)pos >= cap) return kStatusCapacity;
  const int page = p.page_indices[lo + pos / kPage];
  if (page < 0 || page >= p.num_pages) return kStatusPageRange;
  if (p.page_refcounts[page] != 1) return kStatusNotExclusive;
  *page_out = page;
  return 0;
}

// One work-group of 1024 threads.  Each thread checks a strided set of
// tokens; the smallest failing token index wins.
__global__ __launch_bounds__(1024) void append_check_kernel(AppendParams p) {
  __shared__ int first_bad;
  if (threadIdx.x == 0) first_bad = 0x7fffffff;
  __syncthreads();
  int my_t = 0x7fffffff, my_code = 0;
  constexpr int kUnroll = 8;
  for (int base = threadIdx.x; base < p.nnz && my_t == 0x7fffffff; base += 1024 * kUnroll) {
    int codes[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = base + u * 1024;
      int page;
      codes[u] = t < p.nnz ? check_token(p, t, &page) : 0;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (codes[u] != 0 && my_t == 0x7fffffff) { my_t = base + u * 1024; my_code = codes[u]; }
  }
  if (my_t != 0x7fffffff) atomicMin(&first_bad, my_t);
  __syncthreads();
  if (first_bad == 0x7fffffff) {
    if (threadIdx.x == 0) { p.status[0] = 0; p.status[1] = -1; }
  } else if (my_t == first_bad) {
    p.status[0] = my_code;
    p.status[1] = my_t;
  }
}

// float(x) for the 8 bf16 of a 16-byte chunk
__device__ __forceinline__ void unpack8(u32x4_t w, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(w[i]); x[2 * i + 1] = bf16_hi(w[i]); }
}

// Round-to-nearest-even double -> bf16 for results in bf16's normal range,
// from the double's bit fields; anything else takes the general routine.
__device__ __forceinline__ uint32_t bf16_rne(double y) {
  const uint64_t u = __double_as_longlong(y);
  const uint32_t hw = (uint32_t)(u >> 32);
  const uint32_t lw = (uint32_t)u;
  uint32_t field = (hw >> 13) & 0x3ffffu;            // 11 exponent + 7 fraction bits
  const uint32_t rb = (hw >> 12) & 1u;
  const uint32_t sticky = ((hw & 0xfffu) | lw) != 0u;
  field += rb & (sticky | (field & 1u));
  const int e = (int)(field >> 7) - 896;
  if (e >= 1 && e <= 254) return ((hw >> 16) & 0x8000u) | ((uint32_t)e << 7) | (field & 0x7fu);
  return bf16_from_double_rne(y);
}

// Rotate one 8-pair chunk: x1 = dims [8f, 8f+8), x2 = dims [64+8f, 64+8f+8).
__device__ __forceinline__ void rotate_chunk(u32x4_t w1, u32x4_t w2, const double* c,
                                             const double* s, u32x4_t* out1, u32x4_t* out2) {
  float x1[8], x2[8];
  unpack8(w1, x1);
  unpack8(w2, x2);
  uint32_t y1[8], y2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double a = x1[i], bb = x2[i];
    y1[i] = bf16_rne(a * c[i] - bb * s[i]);
    y2[i] = bf16_rne(bb * c[i] + a * s[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    (*out1)[i] = y1[2 * i] | (y1[2 * i + 1] << 16);
    (*out2)[i] = y2[2 * i] | (y2[2 * i + 1] << 16);
  }
}

// Grid-stride over tokens, one wave per token at a time.  Lane l evaluates
// the sin/cos of frequency l and shares it through a wave-private LDS slot;
// lane l then rotates the frequency chunk f = l % 8 (frequencies 8f .. 8f+7)
// of every head it handles.
template <int LAYOUT>
__global__ __launch_bounds__(256) void append_rope_kernel(AppendParams p) {
  __shared__ double cs[4][64][2];
  if (p.status[0] != 0) return;  // all-or-nothing gate
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int f = lane & 7;
  const int hsub = lane >> 3;  // 0..7
  const int nwaves = gridDim.x * 4;
  for (int t = blockIdx.x * 4 + wave; t < p.nnz; t += nwaves) {
    int page;
    if (check_token(p, t, &page) != 0) continue;  // cannot happen after the check
    const int pos = p.positions[t];
    const int slot = pos & (kPage - 1);
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
    const uint16_t* ki = p.k_in + (int64_t)t * p.hkv * kHeadDim;
    const uint16_t* vi = p.v_in + (int64_t)t * p.hkv * kHeadDim;
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
  hipLaunchKernelGGL(append_check_kernel, dim3(1), dim3(1024), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nnz == 0) return e;
  int blocks = (a.nnz + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (a.layout == 0)
    hipLaunchKernelGGL(append_rope_kernel<0>, dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(append_rope_kernel<1>, dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace oxa
