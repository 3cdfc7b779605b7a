// Causal (or full) prefill over ragged or paged K/V on gfx950.
//
// Operator contract: "FlashInfer parity matrix", section "Admitted attention
// matrix" (rows Ragged causal prefill and Paged causal prefill: BF16, head dim
// 128, page size 16, F32 softmax state; short and long MHA, MQA and GQA) and
// section "Dispatch limits" (the pages pick among several NVIDIA kernels by
// average KV length; this library runs one matrix-core kernel for every
// shape, with the tile shape fixed by the head grouping).
//
// Work decomposition (this design): a work-group owns 256 (query row, q head)
// columns that read the same kv head - BM = 256 / G rows of the G = Hq / Hkv
// heads of one group - so each K/V tile staged in LDS serves all of them.
// Eight waves take 32 columns each.  Per 64-key tile a wave forms
// S^T = K * Q^T (16 x v_mfma_f32_32x32x16_bf16, K from LDS, Q^T resident in
// registers), masks only where the tile crosses the causal diagonal or the
// sequence end, updates the f32 online softmax, and accumulates
// O^T = V^T * P^T (16 more MFMAs; V^T through the LDS transpose read, P^T
// straight from the score registers).  Tiles are scheduled longest-first:
// the query-tile index is the slowest grid dimension, counted from the end.
#include "device_common.h"
#include "kernels.h"

namespace oxa {
namespace {

constexpr int kStatusPageRange = 16;
constexpr int kStatusIndptr = 17;
constexpr int kStatusSeqLen = 18;
constexpr int kStatusCausal = 19;

constexpr int kBN = 64;              // keys per tile
constexpr int kNW = 8;               // waves per work-group
constexpr int kCols = kNW * 32;      // (row, head) columns per work-group
constexpr int kRow = kHeadDim + 8;   // LDS row stride (bf16), 16-byte pad
constexpr int kTileElems = kBN * kRow;

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* seq_lens;
  uint16_t* o;
  float* lse;
  int32_t* status;
  int32_t batch, nnz_qo, nnz_kv, hq, hkv, group, gwg, bm, head_tiles, num_tiles;
  int32_t max_qo_len, max_kv_len, causal, num_pages, num_page_entries;
  float scale_log2;
};

struct SeqInfo {
  int q0, qlen;      // query rows [q0, q0 + qlen) of the packed q / o
  int kbase, klen;   // ragged: first packed key row; paged: first page entry
  int code;          // status code (0 = valid)
  bool paged_ok;     // paged: page range check still to do
};

template <bool PAGED>
__device__ __forceinline__ SeqInfo seq_info(const PrefillParams& p, int b) {
  SeqInfo s;
  const int q0 = p.qo_indptr[b], q1 = p.qo_indptr[b + 1];
  s.q0 = q0;
  s.qlen = q1 - q0;
  s.code = 0;
  if (!PAGED) {
    const int k0 = p.kv_indptr[b], k1 = p.kv_indptr[b + 1];
    s.kbase = k0;
    s.klen = k1 - k0;
    if (q0 < 0 || q1 < q0 || q1 > p.nnz_qo || k0 < 0 || k1 < k0 || k1 > p.nnz_kv)
      s.code = kStatusIndptr;
    else if (s.qlen > p.max_qo_len || s.klen > p.max_kv_len || (s.qlen > 0 && s.klen < 1))
      s.code = kStatusSeqLen;
    else if (p.causal && s.qlen > s.klen)
      s.code = kStatusCausal;
  } else {
    const int p0 = p.page_indptr[b], p1 = p.page_indptr[b + 1];
    const int n = p.seq_lens[b];
    s.kbase = p0;
    s.klen = n;
    if (q0 < 0 || q1 < q0 || q1 > p.nnz_qo || p0 < 0 || p1 < p0 || p1 > p.num_page_entries)
      s.code = kStatusIndptr;
    else if (s.qlen > p.max_qo_len || n < 0 || n > p.max_kv_len || (s.qlen > 0 && n < 1))
      s.code = kStatusSeqLen;
    else if ((int64_t)(p1 - p0) * kPage < (int64_t)n)
      s.code = kStatusIndptr;
    else if (p.causal && s.qlen > n)
      s.code = kStatusCausal;
  }
  return s;
}

constexpr int kPidWin = 2048;  // page ids staged in LDS per window (paged K/V)

// Issue the loads of K/V tile `kt` (64 keys): thread tid brings the 16-byte
// chunk `tid % 16` of rows tid/16 and tid/16 + 32, so 16 lanes read one whole
// 256-byte row.  Loads are unconditional - straight-line code keeps the wait
// counters exact - and rows that do not exist read a valid stand-in (key 0 of
// the sequence, or page 0); `ok` marks the real rows for store_tile.
template <bool PAGED, int LAYOUT>
__device__ __forceinline__ void load_tile(const PrefillParams& p, const SeqInfo& si, int kvh,
                                          int kt, int tid, const int* pids, int wbase,
                                          u32x4_t* kr, u32x4_t* vr, bool* ok) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = tid + u * (kNW * 64);
    const int row = c >> 4;
    const int piece = c & 15;
    const int key = kt * kBN + row;
    int64_t off;
    if (!PAGED) {
      ok[u] = key < si.klen;
      const int kc = ok[u] ? key : 0;
      off = ((int64_t)(si.kbase + kc) * p.hkv + kvh) * kHeadDim;
    } else {
      const int pid = key < si.klen ? pids[key / kPage - wbase] : -1;
      ok[u] = pid >= 0;
      const int pc = ok[u] ? pid : 0;
      const int slot = key & (kPage - 1);
      off = LAYOUT == 0 ? (((int64_t)pc * kPage + slot) * p.hkv + kvh) * kHeadDim
                        : (((int64_t)pc * p.hkv + kvh) * kPage + slot) * kHeadDim;
    }
    kr[u] = ldg16(p.k + off + piece * 8);
    vr[u] = ldg16(p.v + off + piece * 8);
  }
}

__device__ __forceinline__ void store_tile(uint16_t* ks, uint16_t* vs, int tid, const u32x4_t* kr,
                                           const u32x4_t* vr, const bool* ok) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = tid + u * (kNW * 64);
    const int row = c >> 4;
    const int piece = c & 15;
    const u32x4_t z = u32x4_t{0, 0, 0, 0};
    *reinterpret_cast<u32x4_t*>(ks + row * kRow + piece * 8) = ok[u] ? kr[u] : z;
    *reinterpret_cast<u32x4_t*>(vs + row * kRow + piece * 8) = ok[u] ? vr[u] : z;
  }
}

template <bool PAGED, int LAYOUT>
__global__ __launch_bounds__(kNW * 64) void prefill_kernel(PrefillParams p) {
  __shared__ __align__(16) uint16_t smem[4 * kTileElems];  // K0, V0, K1, V1
  __shared__ int pids[PAGED ? kPidWin : 1];
  const int kvh = blockIdx.x / p.head_tiles;
  const int ht = blockIdx.x - kvh * p.head_tiles;
  const int b = blockIdx.y;
  const int tile = p.num_tiles - 1 - (int)blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int gi = lane >> 5;
  const int g16 = (lane >> 4) & 1;
  const int i16 = lane & 15;

  SeqInfo si = seq_info<PAGED>(p, b);

  if (p.status != nullptr && blockIdx.x == 0 && tile == 0) {
    int code = si.code;
    if (PAGED && code == 0) {
      const int need = (si.klen + kPage - 1) / kPage;
      int bad = 0;
      for (int i = tid; i < need; i += kNW * 64) {
        const int pid = p.page_indices[si.kbase + i];
        bad |= (pid < 0 || pid >= p.num_pages);
      }
      if (__syncthreads_or(bad)) code = kStatusPageRange;
    }
    if (tid == 0) p.status[b] = code;
  }
  if (si.code != 0) return;
  const int r0 = tile * p.bm;
  if (r0 >= si.qlen) return;
  const int rows_here = min(p.bm, si.qlen - r0);
  const int offset = si.klen - si.qlen;  // bottom-right causal alignment
  const int kv_end = p.causal ? min(si.klen, r0 + rows_here + offset) : si.klen;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // this lane's column: (row, head) pair
  const int pair = wave * 32 + col;
  const int prow = pair / p.gwg;
  const int phead_t = pair - prow * p.gwg;
  const int head_in_group = ht * p.gwg + phead_t;
  const bool col_ok = prow < rows_here && pair < p.bm * p.gwg && head_in_group < p.group;
  const int qrow = r0 + prow;                  // row index within the sequence
  const int head = kvh * p.group + head_in_group;
  const int row_lim = qrow + offset;           // last visible key (causal)

  u32x4_t qf[8];
  if (col_ok) {
    const uint16_t* qp = p.q + ((int64_t)(si.q0 + qrow) * p.hq + head) * kHeadDim + gi * 64;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = ldg16(qp + 8 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = u32x4_t{0, 0, 0, 0};
  }

  f32x16_t acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) acc[d] = f32x16_t{};
  float m = -INFINITY, lsum = 0.f;
  // smallest visible-key limit among the work-group's rows: tiles past it need masks
  const int wg_min_lim = r0 + offset;

  // Paged K/V: the sequence's page ids for keys [0, kv_end), staged per window
  // of kPidWin pages (invalid ids become -1).
  const int npages_need = (kv_end + kPage - 1) / kPage;
  auto stage_pids = [&](int wbase) {
    for (int i = tid; i < kPidWin; i += kNW * 64) {
      const int pg = wbase + i;
      int v = -1;
      if (pg < npages_need) {
        const int pid = p.page_indices[si.kbase + pg];
        v = (pid >= 0 && pid < p.num_pages) ? pid : -1;
      }
      pids[i] = v;
    }
  };
  constexpr int kTilesPerWin = kPidWin * kPage / kBN;
  int wbase = 0;
  if (PAGED) stage_pids(0);
  __syncthreads();

  u32x4_t kr[2], vr[2];
  bool okr[2];
  if (ntiles > 0) {
    load_tile<PAGED, LAYOUT>(p, si, kvh, 0, tid, pids, wbase, kr, vr, okr);
    store_tile(smem, smem + kTileElems, tid, kr, vr, okr);
  }
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const uint16_t* ks = smem + (kt & 1) * 2 * kTileElems;
    const uint16_t* vs = ks + kTileElems;
    if (PAGED && kt + 1 < ntiles && (kt + 1) % kTilesPerWin == 0) {
      // the next tile starts a new page-id window (every waves' reads of the
      // current window are done: only tile kt+1 uses page ids from here on)
      wbase = (kt + 1) / kTilesPerWin * kPidWin;
      __syncthreads();
      stage_pids(wbase);
      __syncthreads();
    }
    if (kt + 1 < ntiles) load_tile<PAGED, LAYOUT>(p, si, kvh, kt + 1, tid, pids, wbase, kr, vr, okr);

    // S^T[key][col] for the 64 keys of the tile: 2 key blocks x 8 k-steps
    f32x16_t s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16_t{};
      const uint16_t* krow = ks + (mb * 32 + col) * kRow + gi * 64;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(krow + 8 * st);
        s[mb] = mfma_32x32x16(a, qf[st], s[mb]);
      }
    }

    const int key0 = kt * kBN;
    const bool need_mask = (key0 + kBN > si.klen) || (p.causal && key0 + kBN - 1 > wg_min_lim);
    float mt = -INFINITY;
    if (need_mask) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + mb * 32 + 8 * (r >> 2) + 4 * gi + (r & 3);
          const bool vis = key < si.klen && (!p.causal || key <= row_lim);
          s[mb][r] = vis ? s[mb][r] * p.scale_log2 : -INFINITY;
          mt = fmaxf(mt, s[mb][r]);
        }
    } else {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[mb][r] *= p.scale_log2;
          mt = fmaxf(mt, s[mb][r]);
        }
    }
    mt = pair_max32(mt);
    const float mnew = fmaxf(m, mt);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    float psum = 0.f;
    uint32_t pk[16];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = exp2f(s[mb][r] - muse);
        const float p1 = exp2f(s[mb][r + 1] - muse);
        psum += p0 + p1;
        pk[mb * 8 + (r >> 1)] = pack_bf16x2(p0, p1);
      }
    if (__builtin_amdgcn_ballot_w64(mnew != m) != 0) {  // rescale only when a max moved
      const float corr = exp2f(m - muse);
      lsum *= corr;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[d][r] *= corr;
    }
    lsum += psum;
    m = mnew;

    // O^T += V^T * P^T over 4 k-steps of 16 keys
#pragma unroll
    for (int ks4 = 0; ks4 < 4; ++ks4) {
      const u32x4_t pf = u32x4_t{pk[4 * ks4], pk[4 * ks4 + 1], pk[4 * ks4 + 2], pk[4 * ks4 + 3]};
      const uint16_t* vrow = vs + (16 * ks4 + 4 * gi + (i16 >> 2)) * kRow + 16 * g16 + 4 * (i16 & 3);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const u32x2_t a0 = lds_read_tr16(vrow + 32 * d);
        const u32x2_t a1 = lds_read_tr16(vrow + 8 * kRow + 32 * d);
        acc[d] = mfma_32x32x16(u32x4_t{a0[0], a0[1], a1[0], a1[1]}, pf, acc[d]);
      }
    }

    if (kt + 1 < ntiles) {
      uint16_t* kn = smem + ((kt + 1) & 1) * 2 * kTileElems;
      store_tile(kn, kn + kTileElems, tid, kr, vr, okr);
    }
    __syncthreads();
  }

  lsum = pair_sum32(lsum);
  if (!col_ok) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  uint16_t* orow = p.o + ((int64_t)(si.q0 + qrow) * p.hq + head) * kHeadDim;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      const int dd = 32 * d + 8 * (r >> 2) + 4 * gi;
      u32x2_t w;
      w[0] = pack_bf16x2(acc[d][r] * inv, acc[d][r + 1] * inv);
      w[1] = pack_bf16x2(acc[d][r + 2] * inv, acc[d][r + 3] * inv);
      *reinterpret_cast<u32x2_t*>(orow + dd) = w;
    }
  if (gi == 0 && p.lse != nullptr)
    p.lse[(int64_t)(si.q0 + qrow) * p.hq + head] =
        lsum > 0.f ? (m + __log2f(lsum)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream) {
  PrefillParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.qo_indptr = a.qo_indptr;
  p.kv_indptr = a.kv_indptr;
  p.page_indptr = a.page_indptr;
  p.page_indices = a.page_indices;
  p.seq_lens = a.seq_lens;
  p.o = a.o;
  p.lse = a.lse;
  p.status = a.status;
  p.batch = a.batch;
  p.nnz_qo = a.nnz_qo;
  p.nnz_kv = a.nnz_kv;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.group = a.hq / a.hkv;
  p.gwg = p.group < kCols ? p.group : kCols;
  p.bm = kCols / p.gwg;
  p.head_tiles = (p.group + p.gwg - 1) / p.gwg;
  p.num_tiles = (a.max_qo_len + p.bm - 1) / p.bm;
  p.max_qo_len = a.max_qo_len;
  p.max_kv_len = a.max_kv_len;
  p.causal = a.causal;
  p.num_pages = a.num_pages;
  p.num_page_entries = a.num_page_entries;
  p.scale_log2 = a.sm_scale * kLog2e;
  dim3 grid(p.hkv * p.head_tiles, p.batch, p.num_tiles);
  dim3 block(kNW * 64);
  if (!a.paged)
    hipLaunchKernelGGL((prefill_kernel<false, 0>), grid, block, 0, stream, p);
  else if (a.layout == 0)
    hipLaunchKernelGGL((prefill_kernel<true, 0>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<true, 1>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace oxa
