// Paged batch decode on gfx950: one query token per sequence over its paged
// KV cache, with optional split-K over explicit KV partitions and a separate
// log-sum-exp merge kernel.
//
// Operator contract: "FlashInfer parity matrix", section "Admitted attention
// matrix" (rows Paged batch decode and Single decode split-K: MHA, MQA and
// GQA, mixed lengths, page order, read-only page reuse, explicit partitions
// with an F32 partial workspace and a merge; BF16, head dim 128, page size 16,
// F32 softmax state) and section "Domain coverage" (NHD and HND paged decode).
//
// Work decomposition (this design, not the pages'): one work-group per
// (partition, kv head, q-head tile of up to 32 heads, sequence).  Each wave of
// the group walks 32-token blocks (two pages) of the partition and keeps its
// own online-softmax state; the waves are merged through LDS at the end.
//
// Per 32-token block a wave computes S^T = K * Q^T with eight
// v_mfma_f32_32x32x16_bf16 (tokens are the M dimension, the grouped q heads of
// one kv head are N), so every lane's K operand is one contiguous 128-byte run
// of a K row, read straight from HBM into registers.  The result leaves each
// lane with one q head and 16 tokens, so the softmax max needs only an
// in-register reduction and one cross-half lane swap.  The probabilities are
// already in the B-operand layout of the PV product O^T = V^T * P^T; V^T comes
// from the block's V rows staged in LDS through the transpose read.
#include "device_common.h"
#include "kernels.h"

namespace oxa {
namespace {

constexpr int kStatusPageRange = 16;
constexpr int kStatusIndptr = 17;
constexpr int kStatusSeqLen = 18;

constexpr int kVRow = kHeadDim + 8;  // staged V row stride in bf16 (16-byte pad)

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* kp;
  const uint16_t* vp;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* seq_lens;
  uint16_t* o;
  float* lse;
  int32_t* status;
  float* ws_o;
  float* ws_lse;
  int32_t batch, hq, hkv, group, head_tiles;
  int32_t num_pages, num_page_entries, max_seq_len, num_partitions, chunk_pages;
  float scale_log2;
};

template <int LAYOUT>
__device__ __forceinline__ int64_t kv_row(int64_t pid, int slot, int h, int hkv) {
  if (LAYOUT == 0) return ((pid * kPage + slot) * hkv + h) * kHeadDim;  // NHD
  return ((pid * hkv + h) * kPage + slot) * kHeadDim;                   // HND
}

template <int LAYOUT, int NW>
__global__ __launch_bounds__(NW * 64) void paged_decode_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int part = blockIdx.x;
  const int kvh = blockIdx.y / p.head_tiles;
  const int ht = blockIdx.y - kvh * p.head_tiles;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;   // MFMA N index: q head within the tile
  const int gi = lane >> 5;    // which half of the k slots this lane holds

  // ---- sequence metadata (uniform) --------------------------------------
  const int L = p.seq_lens[b];
  const int lo = p.page_indptr[b];
  const int hi = p.page_indptr[b + 1];
  const bool len_ok = L >= 1 && L <= p.max_seq_len;
  const bool ptr_ok = lo >= 0 && hi >= lo && hi <= p.num_page_entries &&
                      (int64_t)(hi - lo) * kPage >= (int64_t)L;
  const bool seq_ok = len_ok && ptr_ok;

  if (p.status != nullptr && part == 0 && blockIdx.y == 0) {
    int code = 0;
    if (!len_ok) {
      code = kStatusSeqLen;
    } else if (!ptr_ok) {
      code = kStatusIndptr;
    } else {
      const int need = (L + kPage - 1) / kPage;
      int bad = 0;
      for (int i = tid; i < need; i += NW * 64) {
        const int pid = p.page_indices[lo + i];
        bad |= (pid < 0 || pid >= p.num_pages);
      }
      if (__syncthreads_or(bad)) code = kStatusPageRange;
    }
    if (tid == 0) p.status[b] = code;
  }

  const int chunk_tokens = p.chunk_pages * kPage;
  const int t0 = part * chunk_tokens;
  const int t1 = seq_ok ? min(t0 + chunk_tokens, L) : t0;
  const int nblk = t1 > t0 ? (t1 - t0 + 31) / 32 : 0;

  // ---- Q^T fragments (B operand), loaded once ---------------------------
  const int ncol = min(32, p.group - ht * 32);  // real q heads in this tile
  const bool col_ok = col < ncol;
  const int head = kvh * p.group + ht * 32 + col;
  u32x4_t qf[8];
  if (col_ok) {
    const uint16_t* qp = p.q + ((int64_t)b * p.hq + head) * kHeadDim + gi * 64;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = ldg16(qp + 8 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = u32x4_t{0, 0, 0, 0};
  }

  f32x16_t acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) acc[d] = f32x16_t{};
  float m = -INFINITY;
  float lsum = 0.f;

  uint16_t* vs = reinterpret_cast<uint16_t*>(smem) + wave * 32 * kVRow;
  const int g16 = (lane >> 4) & 1;  // 16-lane group parity: which 16 columns of a 32-wide d block
  const int i16 = lane & 15;

  for (int blk = wave; blk < nblk; blk += NW) {
    const int tb = t0 + blk * 32;  // first token of the block (page aligned)
    const int lp = lo + tb / kPage;
    const int pidA = p.page_indices[lp];
    const int pidB = (tb + kPage < t1) ? p.page_indices[lp + 1] : -1;
    const bool okA = pidA >= 0 && pidA < p.num_pages;
    const bool okB = (tb + kPage < t1) && pidB >= 0 && pidB < p.num_pages;

    // this lane's load token: block row `col`
    const bool ld_ok = (tb + col < t1) && (col < kPage ? okA : okB);
    u32x4_t kf[8], vf[8];
    if (ld_ok) {
      const int pid = col < kPage ? pidA : pidB;
      const int64_t row = kv_row<LAYOUT>(pid, col & (kPage - 1), kvh, p.hkv) + gi * 64;
#pragma unroll
      for (int s = 0; s < 8; ++s) kf[s] = ldg16(p.kp + row + 8 * s);
#pragma unroll
      for (int s = 0; s < 8; ++s) vf[s] = ldg16(p.vp + row + 8 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 8; ++s) { kf[s] = u32x4_t{0, 0, 0, 0}; vf[s] = u32x4_t{0, 0, 0, 0}; }
    }

    // S^T[token][head] over the 128-wide head dim: 8 k-steps of 16
    f32x16_t s = f32x16_t{};
#pragma unroll
    for (int st = 0; st < 8; ++st) s = mfma_32x32x16(kf[st], qf[st], s);

    // stage V rows (zeros for tokens that do not exist) for the transpose read
#pragma unroll
    for (int st = 0; st < 8; ++st)
      *reinterpret_cast<u32x4_t*>(vs + col * kVRow + gi * 64 + 8 * st) = vf[st];

    // mask, scale into the log2 domain, online softmax update
    float sv[16];
    float mblk = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 8 * (r >> 2) + 4 * gi + (r & 3);
      const bool ok = (tb + t < t1) && (t < kPage ? okA : okB);
      sv[r] = ok ? s[r] * p.scale_log2 : -INFINITY;
      mblk = fmaxf(mblk, sv[r]);
    }
    mblk = pair_max32(mblk);
    const float mnew = fmaxf(m, mblk);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float corr = exp2f(m - muse);
    float psum = 0.f;
    uint32_t pk[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = exp2f(sv[r] - muse);
      const float p1 = exp2f(sv[r + 1] - muse);
      psum += p0 + p1;
      pk[r >> 1] = pack_bf16x2(p0, p1);
    }
    lsum = lsum * corr + psum;
    m = mnew;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] *= corr;

    // O^T[d][head] += V^T[d][token] * P^T[token][head], 2 k-steps x 4 d-blocks
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t pf = u32x4_t{pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
      const uint16_t* vrow = vs + (16 * ks + 4 * gi + (i16 >> 2)) * kVRow + 16 * g16 + 4 * (i16 & 3);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const u32x2_t a0 = lds_read_tr16(vrow + 32 * d);
        const u32x2_t a1 = lds_read_tr16(vrow + 8 * kVRow + 32 * d);
        acc[d] = mfma_32x32x16(u32x4_t{a0[0], a0[1], a1[0], a1[1]}, pf, acc[d]);
      }
    }
  }

  // ---- merge the waves' states through LDS -------------------------------
  lsum = pair_sum32(lsum);
  __syncthreads();  // staging area is reused below
  float* red_m = reinterpret_cast<float*>(smem);         // [NW][32]
  float* red_l = red_m + NW * 32;                         // [NW][32]
  float* red_o = red_l + NW * 32;                         // [NW][128][ncol]
  if (gi == 0) {
    red_m[wave * 32 + col] = m;
    red_l[wave * 32 + col] = lsum;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w * 32 + col]);
  const float Muse = M == -INFINITY ? 0.f : M;
  const float f = exp2f(m - Muse);
  if (col_ok) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dd = 32 * d + 8 * (r >> 2) + 4 * gi + (r & 3);
        red_o[(wave * kHeadDim + dd) * ncol + col] = acc[d][r] * f;
      }
  }
  __syncthreads();
  const bool split = p.num_partitions > 1;
  for (int idx = tid; idx < ncol * kHeadDim; idx += NW * 64) {
    const int c = idx % ncol;
    const int dd = idx / ncol;
    float mc = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mc = fmaxf(mc, red_m[w * 32 + c]);
    const float mcu = mc == -INFINITY ? 0.f : mc;
    float lc = 0.f, oc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      lc += red_l[w * 32 + c] * exp2f(red_m[w * 32 + c] - mcu);
      oc += red_o[(w * kHeadDim + dd) * ncol + c];
    }
    const float val = lc > 0.f ? oc / lc : 0.f;
    const float lse_val = lc > 0.f ? (mc + __log2f(lc)) * kLn2 : -INFINITY;
    const int64_t hrow = (int64_t)b * p.hq + kvh * p.group + ht * 32 + c;
    if (split) {
      const int64_t prow = hrow * p.num_partitions + part;
      p.ws_o[prow * kHeadDim + dd] = val;
      if (dd == 0) p.ws_lse[prow] = lse_val;
    } else {
      p.o[hrow * kHeadDim + dd] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xffffu);
      if (dd == 0 && p.lse != nullptr) p.lse[hrow] = lse_val;
    }
  }
}

// LSE merge of split-K partial states: one 128-thread group per (sequence, q head).
__global__ __launch_bounds__(128) void merge_partials_kernel(const float* ws_o, const float* ws_lse,
                                                             int num_partitions, uint16_t* o,
                                                             float* lse) {
  const int64_t row = blockIdx.x;
  const int d = threadIdx.x;
  const float* lp = ws_lse + row * num_partitions;
  const float* op = ws_o + row * num_partitions * kHeadDim;
  float mx = -INFINITY;
  for (int i = 0; i < num_partitions; ++i) mx = fmaxf(mx, lp[i]);
  const float mu = mx == -INFINITY ? 0.f : mx;
  float wsum = 0.f, acc = 0.f;
  for (int i = 0; i < num_partitions; ++i) {
    const float w = __expf(lp[i] - mu);
    wsum += w;
    acc += w * op[(int64_t)i * kHeadDim + d];
  }
  const float val = wsum > 0.f ? acc / wsum : 0.f;
  o[row * kHeadDim + d] = (uint16_t)(pack_bf16x2(val, 0.f) & 0xffffu);
  if (d == 0 && lse != nullptr) lse[row] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

template <int LAYOUT, int NW>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  const int ncol = p.group < 32 ? p.group : 32;
  const size_t stage = (size_t)NW * 32 * kVRow * sizeof(uint16_t);
  const size_t reduce = (size_t)NW * 64 * sizeof(float) + (size_t)NW * kHeadDim * ncol * sizeof(float);
  const size_t lds = stage > reduce ? stage : reduce;
  dim3 grid(p.num_partitions, p.hkv * p.head_tiles, p.batch);
  hipLaunchKernelGGL((paged_decode_kernel<LAYOUT, NW>), grid, dim3(NW * 64), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode(const DecodeLaunch& a, hipStream_t stream) {
  DecodeParams p;
  p.q = a.q;
  p.kp = a.k_pages;
  p.vp = a.v_pages;
  p.page_indptr = a.page_indptr;
  p.page_indices = a.page_indices;
  p.seq_lens = a.seq_lens;
  p.o = a.o;
  p.lse = a.lse;
  p.status = a.status;
  p.ws_o = a.ws_o;
  p.ws_lse = a.ws_lse;
  p.batch = a.batch;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.group = a.hq / a.hkv;
  p.head_tiles = (p.group + 31) / 32;
  p.num_pages = a.num_pages;
  p.num_page_entries = a.num_page_entries;
  p.max_seq_len = a.max_seq_len;
  p.num_partitions = a.num_partitions;
  p.chunk_pages = a.chunk_pages;
  p.scale_log2 = a.sm_scale * kLog2e;
  hipError_t e;
  if (a.layout == 0)
    e = launch_decode_t<0, 8>(p, stream);
  else
    e = launch_decode_t<1, 8>(p, stream);
  if (e != hipSuccess || a.num_partitions == 1) return e;
  hipLaunchKernelGGL(merge_partials_kernel, dim3(a.batch * a.hq), dim3(kHeadDim), 0, stream,
                     a.ws_o, a.ws_lse, a.num_partitions, a.o, a.lse);
  return hipGetLastError();
}

}  // namespace oxa
