// Load-balanced paged decode on gfx950: equal page ranges per work-group.
//
// Operator contract: "FlashInfer parity matrix", section "Admitted attention
// matrix" (rows Paged batch decode and Single decode split-K: MHA, MQA and
// GQA, mixed lengths, page order, read-only page reuse, explicit partitions
// with an F32 partial workspace and a merge; BF16, head dim 128, page size 16,
// F32 softmax state) and section "Domain coverage" (NHD and HND paged decode).
// The result is the same attention as the per-(sequence, kv head) kernel;
// only the division of the work differs (this design, not the pages').
//
// Decode reads every K/V row once, so it is bound by HBM bandwidth, and one
// compute unit streams at most ~50 GB/s: a long sequence held by one
// work-group sets the time of a whole mixed-length batch.  Here the pages of
// all units (a unit is a sequence, or one of its explicit partitions) are laid
// end to end and cut into G equal ranges, one per work-group (times the
// stream-set groups below), so every compute unit streams the same bytes.  A
// unit that a range boundary cuts yields partial states (normalised output and
// natural-log lse per q head), which a second kernel merges; a unit inside one
// range is written directly.
//
// A stream is a (kv head, tile of up to 16 grouped q heads) pair and a stream
// set holds the streams of one kv head that a wave computes together (one
// tile when a kv head has a single tile, else two).  A work-group of 8 waves
// (two per SIMD) serves up to 8 sets; the waves of a set split its 32-token
// blocks (page pairs), merging at the end of each piece.  Each wave pipelines
// its own K/V rows: the next pair's rows are loaded into registers while the
// current pair is computed from the wave's LDS slice, then staged there
// (XOR-swizzled rows), so the loop needs no barrier.  Per pair and stream:
// S^T = K Q^T with 8 v_mfma_f32_16x16x32_bf16 (tokens are M, q heads N; the K
// fragments serve both streams of the set), an online softmax with a lazy
// reference max over the pair's 32 scores, and O^T += V^T P^T with 8 more
// (the 32 tokens are the reduction; V^T through the LDS transpose read).
#include "device_common.h"
#include "kernels.h"

namespace oxa {
namespace {

constexpr int kStatusPageRange = 16;
constexpr int kStatusIndptr = 17;
constexpr int kStatusSeqLen = 18;

constexpr int kNW = 8;                 // waves per work-group
constexpr int kHT = 16;                // q heads per stream (MFMA N)
constexpr int kSets = 8;               // stream sets per work-group at most
constexpr int kHalf = kPage * 256;     // K (or V) rows of one page of one kv head: 4 KB
constexpr int kWaveSlice = 4 * kHalf;  // a wave's K and V rows of a page pair: 16 KB
constexpr int kSlots = 16;             // per-wave stream states merged at a piece end
constexpr int kPidWin = 512;           // page ids staged in LDS at a time

// LDS: the waves' row slices, reused by the piece epilogue (column max and sum
// [kSlots][16], accumulators [kSlots][128][16]); then the unit page starts,
// the page-id window and a small reduction area.
constexpr int kLdsEpi = (2 * kSlots * kHT + kSlots * kHeadDim * kHT) * 4;
constexpr int kLdsUnits = kNW * kWaveSlice > kLdsEpi ? kNW * kWaveSlice : kLdsEpi;
// per unit: first flat page (ustart), page-table entry of its first page
// (uptr) and tokens on its last page (utail)
constexpr int kLdsUptr = kLdsUnits + (kBalancedMaxUnits + 1) * 4;
constexpr int kLdsUtail = kLdsUptr + kBalancedMaxUnits * 4;
constexpr int kLdsPids = kLdsUtail + kBalancedMaxUnits * 4;
constexpr int kLdsRed = kLdsPids + kPidWin * 4;
constexpr int kLdsPinfo = kLdsRed + 64 * 4;  // independent waves: unit | valid tokens << 16
constexpr int kLdsBytes = kLdsPinfo + kPidWin * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one compute unit");

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

struct BalParams {
  const uint16_t* q;
  const uint16_t* kp;
  const uint16_t* vp;
  const int32_t* page_indptr;
  const int32_t* page_indices;
  const int32_t* seq_lens;
  uint16_t* o;
  float* lse;
  int32_t* status;
  float* ws_o;       // partition states [batch][hq][P][128] (P > 1)
  float* ws_lse;     // [batch][hq][P]
  int32_t* meta;     // unit page starts [units + 1], written by work-group 0
  float* piece_o;    // piece states [(G + units)][hq][128]
  float* piece_lse;  // [(G + units)][hq]
  int32_t batch, hq, hkv, group, head_tiles, sets_per_head, total_sets, nsg;
  int32_t num_pages, num_page_entries, max_seq_len, num_partitions, chunk_pages;
  int32_t units, G;
  float scale_log2;
};

__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Byte offset of 16-byte chunk c of token row t in a block of 256-byte rows,
// chunks XOR-swizzled by 2*(t % 8) + (t / 8) % 2: conflict-free for 16 lanes
// reading one chunk of 16 consecutive rows (the K operand), 16 lanes writing
// one row, and the transpose read of consecutive rows x 32 bytes (V^T).
__device__ __forceinline__ int swz(int t, int c) {
  const int sw = ((t & 7) << 1) | ((t >> 3) & 1);
  return (t * 16 + (c ^ sw)) << 4;
}

// Pages of unit u (sequence u / P, partition u % P); 0 if the sequence's
// metadata is invalid (its status then says why and nothing reads its pages).
// Also the page-table entry of the unit's first page and the tokens on its
// last page.
__device__ __forceinline__ int unit_pages(const BalParams& p, int u, int* entry, int* tail) {
  const int b = u / p.num_partitions;
  const int part = u - b * p.num_partitions;
  const int L = p.seq_lens[b];
  const int lo = p.page_indptr[b], hi = p.page_indptr[b + 1];
  const bool ok = L >= 1 && L <= p.max_seq_len && lo >= 0 && hi >= lo &&
                  hi <= p.num_page_entries && (int64_t)(hi - lo) * kPage >= (int64_t)L;
  *entry = lo + part * p.chunk_pages;
  if (!ok) return 0;
  const int need = (L + kPage - 1) / kPage;
  const int n = max(0, min(p.chunk_pages, need - part * p.chunk_pages));
  // the unit's last page is the sequence's last page or a full one
  *tail = part * p.chunk_pages + n == need ? L - (need - 1) * kPage : kPage;
  return n;
}

// Exclusive prefix sum over a[0 .. n) in LDS, a[n] <- total; kNW * 64 threads.
__device__ __forceinline__ void lds_prefix_sum(int* a, int n, int* red, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int per = (n + kNW * 64 - 1) / (kNW * 64);
  const int lo = min(tid * per, n), hi = min(lo + per, n);
  int sum = 0;
  for (int u = lo; u < hi; ++u) sum += a[u];
  int incl = sum;  // inclusive scan over the lanes of the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  int run = incl - sum;
  int total = 0;
  for (int w = 0; w < kNW; ++w) {
    if (w < wave) run += red[w];
    total += red[w];
  }
  __syncthreads();
  for (int u = lo; u < hi; ++u) {
    const int c = a[u];
    a[u] = run;
    run += c;
  }
  if (tid == 0) a[n] = total;
  __syncthreads();
}

__device__ __forceinline__ int range_start(int64_t w, int64_t total, int G) {
  return (int)(w * total / G);
}

__device__ __forceinline__ int range_of(int page, int total, int G) {
  int w = (int)((int64_t)page * G / total);
  while (w + 1 < G && range_start(w + 1, total, G) <= page) ++w;
  while (w > 0 && range_start(w, total, G) > page) --w;
  return w;
}

template <int LAYOUT, int NS, bool NT, bool INDEP>
__global__ __launch_bounds__(kNW * 64) void balanced_decode_kernel(BalParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* ustart = reinterpret_cast<int*>(smem + kLdsUnits);
  int* pids = reinterpret_cast<int*>(smem + kLdsPids);
  int* red = reinterpret_cast<int*>(smem + kLdsRed);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;  // MFMA N index: q head within the stream
  const int gq = lane >> 4;   // quarter of the k slots this lane holds
  const int w = blockIdx.x / p.nsg;      // page range
  const int g = blockIdx.x - w * p.nsg;  // stream-set group

  int* uptr = reinterpret_cast<int*>(smem + kLdsUptr);
  int* utail = reinterpret_cast<int*>(smem + kLdsUtail);

  // The sequences whose status this work-group checks at the end (b = w,
  // w + G, ...; stream-set group 0): the first one's page ids are loaded now,
  // their latency hidden behind the attention work.
  const bool checks = p.status != nullptr && g == 0 && w < p.batch;
  int st_L = 0, st_lo = 0, st_hi = 0, st_pid = 0;
  if (checks) {
    st_L = p.seq_lens[w];
    st_lo = p.page_indptr[w];
    st_hi = p.page_indptr[w + 1];
    const bool ok = st_L >= 1 && st_L <= p.max_seq_len && st_lo >= 0 && st_hi >= st_lo &&
                    st_hi <= p.num_page_entries && (int64_t)(st_hi - st_lo) * kPage >= (int64_t)st_L;
    if (ok && tid < (st_L + kPage - 1) / kPage) st_pid = p.page_indices[st_lo + tid];
  }

  // ---- unit page starts (every work-group derives the same) -------------
  for (int u = tid; u < p.units; u += kNW * 64) {
    int e = 0, t = kPage;
    ustart[u] = unit_pages(p, u, &e, &t);
    uptr[u] = e;
    utail[u] = t;
  }
  __syncthreads();
  lds_prefix_sum(ustart, p.units, red, tid);
  const int total = ustart[p.units];
  if (blockIdx.x == 0)
    for (int u = tid; u <= p.units; u += kNW * 64) p.meta[u] = ustart[u];
  const int s0 = range_start(w, total, p.G);
  const int s1 = range_start(w + 1, total, p.G);

  // ---- this wave's stream set ------------------------------------------------
  // nsets sets here, tgn waves per set (token groups: wave tgi of a set takes
  // the page pairs tgi, tgi + tgn, ... of each piece); waves past
  // nsets * tgn idle but join the barriers.
  const int set0 = g * kSets;
  const int nsets = min(kSets, p.total_sets - set0);
  const int tgn = kNW / nsets;
  const int sl = wave / tgn;
  const int tgi = wave - sl * tgn;
  const bool busy = sl < nsets;
  const int set = set0 + min(sl, nsets - 1);
  const int kvh = set / p.sets_per_head;
  const int tile0 = (set - kvh * p.sets_per_head) * NS;
  int ncol[NS];
  bool col_ok[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int tile = tile0 + i;
    ncol[i] = tile < p.head_tiles ? min(kHT, p.group - tile * kHT) : 0;
    col_ok[i] = busy && col < ncol[i];
  }
  const int row_bytes = (LAYOUT == 0 ? p.hkv * kHeadDim : kHeadDim) * 2;
  const int64_t page_bytes = (int64_t)kPage * p.hkv * kHeadDim * 2;
  const int64_t head_bytes = (int64_t)kvh * (LAYOUT == 0 ? kHeadDim : kPage * kHeadDim) * 2;
  const unsigned char* kb = reinterpret_cast<const unsigned char*>(p.kp) + head_bytes;
  const unsigned char* vb = reinterpret_cast<const unsigned char*>(p.vp) + head_bytes;
  const uint32_t lane_chunk = 16 * (lane & 15);
  unsigned char* kslice = smem + wave * kWaveSlice;  // [pair page][16 rows] K
  unsigned char* vslice = kslice + 2 * kHalf;         // the same for V

  f32x4_t acc[NS][8];
  float m[NS], lsum[NS];
  u32x4_t qf[NS][4];  // Q^T B operand: lane l holds head l % 16, dims 32*kk + 8*(l/16) .. +8

  struct Rows {
    u32x4_t k[2][4];  // [pair page][row quad]
    u32x4_t v[2][4];
  };
  // Rows of the pages pid[0], pid[1] of a pair: lane l loads 16 bytes of
  // rows 4*q4 + l/16.  Rows past last[pg] (the last token of the page)
  // re-read that row (unused slots may hold anything, NaN included, and a
  // zero weight times NaN would still be NaN in the product); a pair of one
  // page passes that page twice with last 0.  An invalid page id reads page 0
  // (the sequence's status then says so).
  auto issue_pages = [&](const int (&pid_in)[2], const int (&last_in)[2], Rows& r) {
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
      const int pid = __builtin_amdgcn_readfirstlane(max(pid_in[pg], 0));
      const int last = __builtin_amdgcn_readfirstlane(last_in[pg]);
      const unsigned char* ka = kb + pid * page_bytes;
      const unsigned char* va = vb + pid * page_bytes;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint32_t off = (uint32_t)(min(4 * q4 + gq, last) * row_bytes) + lane_chunk;
        const u32x4_t* kp4 = reinterpret_cast<const u32x4_t*>(ka + off);
        const u32x4_t* vp4 = reinterpret_cast<const u32x4_t*>(va + off);
        if constexpr (NT) {
          r.k[pg][q4] = __builtin_nontemporal_load(kp4);
          r.v[pg][q4] = __builtin_nontemporal_load(vp4);
        } else {
          r.k[pg][q4] = *kp4;
          r.v[pg][q4] = *vp4;
        }
      }
    }
  };
  auto stage = [&](const Rows& r) {
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int off = pg * kHalf + swz(4 * q4 + gq, col);
        *reinterpret_cast<u32x4_t*>(kslice + off) = r.k[pg][q4];
        *reinterpret_cast<u32x4_t*>(vslice + off) = r.v[pg][q4];
      }
  };
  // attention over the staged pair: valid0 / valid1 tokens of its pages exist
  auto compute = [&](int valid0, int valid1) {
    // S^T[token][head] per page: A operand of lane l is token l % 16, dims
    // 32*kk + 8*(l/16) .. +8; one K fragment serves every stream of the set
    f32x4_t s[NS][2];
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int pg = 0; pg < 2; ++pg) s[i][pg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const u32x4_t kf =
            *reinterpret_cast<const u32x4_t*>(kslice + pg * kHalf + swz(col, 4 * kk + gq));
#pragma unroll
        for (int i = 0; i < NS; ++i) s[i][pg] = mfma_16x16x32(kf, qf[i][kk], s[i][pg]);
      }
    // P^T B operand of the 16x16x32 product: k slot 8*gq + j of lane l is
    // token 4*gq + j of page 0 (j < 4) or 4*gq + j - 4 of page 1, exactly the
    // scores this lane holds
    u32x4_t pf[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      float sv[8];
      float mraw = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sv[e] = (4 * gq + e < valid0) ? s[i][0][e] : -INFINITY;
        sv[4 + e] = (4 * gq + e < valid1) ? s[i][1][e] : -INFINITY;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) mraw = fmaxf(mraw, sv[e]);
      mraw = pair_max32(pair_max16(mraw));
      // (a pair with no visible token keeps -inf, also for a zero scale)
      const float mblk = mraw == -INFINITY ? -INFINITY : mraw * p.scale_log2;
      // Lazy reference max: it moves only when exceeded by more than 2^8
      // (the reference cancels in o = acc / l).
      if (__builtin_amdgcn_ballot_w64(mblk > m[i] + 8.f) != 0) {
        const float mnew = mblk > m[i] + 8.f ? mblk : m[i];
        const float corr = fast_exp2(m[i] - mnew);  // 0 while m is still -inf
        lsum[i] *= corr;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[i][d] *= corr;
        m[i] = mnew;
      }
      const float muse = m[i] == -INFINITY ? 0.f : m[i];
      float pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // masked tokens weigh exactly 0 (fmaf(-inf, 0, x) is NaN)
        const float v = fast_exp2(fmaf(sv[e], p.scale_log2, -muse));
        pr[e] = sv[e] == -INFINITY ? 0.f : v;
      }
      lsum[i] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
      pf[i] = u32x4_t{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                      pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
    }
    // O^T[d][head] += V^T[d][token] P^T[token][head], 8 d-blocks of 16; the
    // V^T fragment of lane l (dim 16*d + l % 16, k slots 8*(l/16) .. +8) is
    // two transpose reads, one per page: lanes 4e..4e+3 of each 16-lane group
    // address token row 4*gq + e, 8 bytes each of the 32-byte dim segment
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int off = swz(4 * gq + (col >> 2), 2 * d + ((col & 3) >> 1)) + 8 * (col & 1);
      const u32x2_t a0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(vslice + off));
      const u32x2_t a1 = lds_read_tr16(reinterpret_cast<const uint16_t*>(vslice + kHalf + off));
      const u32x4_t vf = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
      for (int i = 0; i < NS; ++i) acc[i][d] = mfma_16x16x32(vf, pf[i], acc[i][d]);
    }
  };

  // open a piece of unit u: this wave's Q fragments of sequence u / P and an
  // empty softmax state
  auto start_piece = [&](int u) {
    const int b = u / p.num_partitions;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (col_ok[i]) {
        const int head = kvh * p.group + (tile0 + i) * kHT + col;
        const uint16_t* qp = p.q + ((int64_t)b * p.hq + head) * kHeadDim + 8 * gq;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[i][kk] = ldg16(qp + 32 * kk);
      } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qf[i][kk] = u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[i][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m[i] = -INFINITY;
      lsum[i] = 0.f;
    }
  };
  // Write this wave's state of the finished piece of unit u (a wave that
  // owns its set alone): the normalised output and lse per q head, to o and
  // lse (a whole unit, P == 1), to the partition state (a whole unit, P > 1)
  // or to the piece slot.  Lane (c, g) holds dims 16*d + 4*g .. +4 of head c.
  auto finish_piece_wave = [&](int u) {
    const int us = ustart[u], ue = ustart[u + 1];
    const int pa = max(s0, us), pb = min(s1, ue);
    const bool whole = pa == us && pb == ue;
    const int slot = pa == s0 ? w : p.G + u;
    const int b = u / p.num_partitions;
    const int part = u - b * p.num_partitions;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const float lt = pair_sum32(pair_sum16(lsum[i]));
      if (!col_ok[i]) continue;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const float lse_val = lt > 0.f ? (m[i] + __log2f(lt)) * kLn2 : -INFINITY;
      const int head = kvh * p.group + (tile0 + i) * kHT + col;
      const int64_t hrow = (int64_t)b * p.hq + head;
      if (whole && p.num_partitions == 1) {
        uint16_t* dst = p.o + hrow * kHeadDim + 4 * gq;
#pragma unroll
        for (int d = 0; d < 8; ++d)
          *reinterpret_cast<u32x2_t*>(dst + 16 * d) =
              u32x2_t{pack_bf16x2(acc[i][d][0] * inv, acc[i][d][1] * inv),
                      pack_bf16x2(acc[i][d][2] * inv, acc[i][d][3] * inv)};
        if (gq == 0 && p.lse != nullptr) p.lse[hrow] = lse_val;
      } else {
        float* dst;
        float* ldst;
        if (whole) {
          const int64_t prow = hrow * p.num_partitions + part;
          dst = p.ws_o + prow * kHeadDim;
          ldst = p.ws_lse + prow;
        } else {
          const int64_t srow = (int64_t)slot * p.hq + head;
          dst = p.piece_o + srow * kHeadDim;
          ldst = p.piece_lse + srow;
        }
#pragma unroll
        for (int d = 0; d < 8; ++d)
          *reinterpret_cast<f32x4_t*>(dst + 16 * d + 4 * gq) = acc[i][d] * inv;
        if (gq == 0) *ldst = lse_val;
      }
    }
  };

  // Several waves per set: merge their states of the finished piece of unit
  // u through LDS and write them.  Every wave of the work-group calls it at
  // the same piece end.  LDS (the row slices, free by then): per wave-state
  // slot ls the column max and sum [16] and the accumulator laid out
  // [d][e][g][c] for lane (c, g)'s acc[d][e], so the 64 lanes of a store write
  // 64 consecutive words.
  auto finish_piece_shared = [&](int u) {
    const int us = ustart[u], ue = ustart[u + 1];
    const int pa = max(s0, us), pb = min(s1, ue);
    const bool whole = pa == us && pb == ue;
    const int slot = pa == s0 ? w : p.G + u;
    const int b = u / p.num_partitions;
    const int part = u - b * p.num_partitions;
    float* red_m = reinterpret_cast<float*>(smem);  // [kSlots][16]
    float* red_l = red_m + kSlots * kHT;            // [kSlots][16]
    float* red_o = red_l + kSlots * kHT;            // [kSlots][8][4][4][16]
    __syncthreads();  // every wave is done with its row slice
    if (busy) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (ncol[i] == 0) continue;
        const int ls = (sl * NS + i) * tgn + tgi;
        const float lt = pair_sum32(pair_sum16(lsum[i]));
        if (gq == 0) {
          red_m[ls * kHT + col] = m[i];
          red_l[ls * kHT + col] = lt;
        }
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
          for (int e = 0; e < 4; ++e) red_o[((ls * 8 + d) * 4 + e) * 64 + lane] = acc[i][d][e];
      }
    }
    __syncthreads();
    // thread (k, i, c, dc): set k, its stream i, q head c, dims 8*dc .. +8
    for (int item = tid; item < nsets * NS * kHT * 16; item += kNW * 64) {
      const int k = item / (NS * kHT * 16);
      const int i = (item / (kHT * 16)) % NS;
      const int c = (item / 16) % kHT;
      const int dc = item % 16;
      const int setk = set0 + k;
      const int kvhk = setk / p.sets_per_head;
      const int tile = (setk - kvhk * p.sets_per_head) * NS + i;
      if (tile >= p.head_tiles || c >= min(kHT, p.group - tile * kHT)) continue;
      const int lbase = (k * NS + i) * tgn;
      float M = -INFINITY;
      for (int t = 0; t < tgn; ++t) M = fmaxf(M, red_m[(lbase + t) * kHT + c]);
      const float Muse = M == -INFINITY ? 0.f : M;
      float Lt = 0.f;
      float val[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int t = 0; t < tgn; ++t) {
        const float f = fast_exp2(red_m[(lbase + t) * kHT + c] - Muse);
        Lt += red_l[(lbase + t) * kHT + c] * f;
        // dims 8*dc + j: d = dc / 2, g = 2 * (dc % 2) + j / 4, e = j % 4
        const float* ro = red_o + (((lbase + t) * 8 + (dc >> 1)) * 4) * 64 + (2 * (dc & 1)) * 16 + c;
#pragma unroll
        for (int j = 0; j < 8; ++j) val[j] += ro[(j & 3) * 64 + (j >> 2) * 16] * f;
      }
      const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) val[j] *= inv;
      const float lse_val = Lt > 0.f ? (M + __log2f(Lt)) * kLn2 : -INFINITY;
      const int head = kvhk * p.group + tile * kHT + c;
      const int64_t hrow = (int64_t)b * p.hq + head;
      if (whole && p.num_partitions == 1) {
        *reinterpret_cast<u32x4_t*>(p.o + hrow * kHeadDim + 8 * dc) =
            u32x4_t{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3]),
                    pack_bf16x2(val[4], val[5]), pack_bf16x2(val[6], val[7])};
        if (dc == 0 && p.lse != nullptr) p.lse[hrow] = lse_val;
      } else {
        float* dst;
        float* ldst;
        if (whole) {  // partition state in the documented workspace
          const int64_t prow = hrow * p.num_partitions + part;
          dst = p.ws_o + prow * kHeadDim;
          ldst = p.ws_lse + prow;
        } else {      // piece state for the merge kernel
          const int64_t srow = (int64_t)slot * p.hq + head;
          dst = p.piece_o + srow * kHeadDim;
          ldst = p.piece_lse + srow;
        }
        *reinterpret_cast<f32x4_t*>(dst + 8 * dc) = f32x4_t{val[0], val[1], val[2], val[3]};
        *reinterpret_cast<f32x4_t*>(dst + 8 * dc + 4) = f32x4_t{val[4], val[5], val[6], val[7]};
        if (dc == 0) *ldst = lse_val;
      }
    }
    __syncthreads();  // the slices are free for the next pair's rows
  };

  // ---- the pages of this range, a window of descriptors at a time.
  // Descriptors (page id, and unit | valid tokens << 16) of up to kPidWin
  // pages are staged together.  The range's pieces (one per unit it touches)
  // are walked in order by every wave; within a piece the page pairs
  // (2k, 2k+1 from the piece's start in the window) go to the set's waves in
  // turn (pair k to wave tgi = k mod tgn).  A wave's next pair is prefetched
  // whatever piece it lies in, so piece ends do not drain the load pipeline.
  int* pinfo = reinterpret_cast<int*>(smem + kLdsPinfo);
  for (int w0 = s0; w0 < s1; w0 += kPidWin) {
    const int wend = min(s1, w0 + kPidWin);
    const int wlen = wend - w0;
    __syncthreads();  // the previous window's descriptors are free
    for (int i = tid; i < wlen; i += kNW * 64) {
      const int f = w0 + i;
      int lo = 0, hi = p.units - 1;  // last unit starting at or before f
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ustart[mid] <= f) lo = mid; else hi = mid - 1;
      }
      const int uu = lo;  // unit_pages > 0 for the unit holding f
      const int pid = p.page_indices[uptr[uu] + (f - ustart[uu])];
      pids[i] = (pid >= 0 && pid < p.num_pages) ? pid : -1;
      pinfo[i] = uu | ((f == ustart[uu + 1] - 1 ? utail[uu] : kPage) << 16);
    }
    __syncthreads();
    auto unit_at = [&](int i) { return pinfo[i] & 0xffff; };
    // window-local end of the piece that starts at window page i
    auto piece_end = [&](int i) { return min(wend, ustart[unit_at(i) + 1]) - w0; };
    // pair k of the piece starting at pa (its end pe), or else pair tgi of a
    // later piece; false past the window
    auto find = [&](int& pa, int& k, int& pe) {
      while (pa < wlen) {
        pe = piece_end(pa);
        if (2 * k < pe - pa) return true;
        pa = pe;
        k = tgi;
      }
      return false;
    };
    auto issue_item = [&](int pa, int k, int pe, Rows& r) {
      const int i = pa + 2 * k;
      const int len = i + 1 < pe ? 2 : 1;
      int pid2[2] = {pids[i], pids[i + len - 1]};
      int last2[2] = {(pinfo[i] >> 16) - 1, len == 2 ? (pinfo[i + 1] >> 16) - 1 : 0};
      issue_pages(pid2, last2, r);
    };
    Rows r;
    int cpa = 0, ck = tgi, cpe = 0;  // this wave's current pair
    bool have = busy && find(cpa, ck, cpe);
    if (have) issue_item(cpa, ck, cpe, r);
    for (int pa = 0; pa < wlen;) {
      const int u = unit_at(pa);
      const int pe = piece_end(pa);
      // a piece already open at the window start goes on with its state
      if (!(pa == 0 && w0 > s0 && ustart[u] < w0)) start_piece(u);
      while (have && cpa == pa) {
        int npa = cpa, nk = ck + tgn, npe = 0;
        const bool hn = find(npa, nk, npe);
        stage(r);
        if (hn) issue_item(npa, nk, npe, r);
        const int i = cpa + 2 * ck;
        compute(pinfo[i] >> 16, i + 1 < cpe ? pinfo[i + 1] >> 16 : 0);
        cpa = npa;
        ck = nk;
        cpe = npe;
        have = hn;
      }
      if (w0 + pe == min(s1, ustart[u + 1])) {  // the piece ends in this window
        if constexpr (INDEP)
          finish_piece_wave(u);
        else
          finish_piece_shared(u);
      }
      pa = pe;
    }
  }

  // ---- per-sequence status: work-group w (set group 0) checks the
  // sequences b = w, w + G, ... after its attention work
  if (checks) {
    for (int b = w; b < p.batch; b += p.G) {
      const bool first = b == w;
      const int L = first ? st_L : p.seq_lens[b];
      const int lo = first ? st_lo : p.page_indptr[b];
      const int hi = first ? st_hi : p.page_indptr[b + 1];
      int code = 0;
      if (!(L >= 1 && L <= p.max_seq_len)) {
        code = kStatusSeqLen;
      } else if (!(lo >= 0 && hi >= lo && hi <= p.num_page_entries &&
                   (int64_t)(hi - lo) * kPage >= (int64_t)L)) {
        code = kStatusIndptr;
      } else {
        const int need = (L + kPage - 1) / kPage;
        int bad = 0;
        for (int i = tid; i < need; i += kNW * 64) {
          const int pid = first && i == tid ? st_pid : p.page_indices[lo + i];
          bad |= (pid < 0 || pid >= p.num_pages);
        }
        if (__syncthreads_or(bad)) code = kStatusPageRange;
      }
      if (tid == 0) p.status[b] = code;
    }
  }
}

// Merge kernel: one work-group of 8 lane groups (32 lanes, 4 floats of the
// 128-dim row each) per row, a (sequence, q head).  The groups split the
// row's partitions (units) and, when there are fewer than 8, each unit's
// pieces as well, so long chains of pieces are folded in parallel: gpp =
// 8 / P groups per partition (1 when P >= 8, the partitions then taken 8 at a
// time).  A single unit of at most 8 pieces is folded by group 0 alone.  A unit cut by range boundaries has pieces in the ranges
// w0 .. w1 that hold pages (first piece: slot w0 if the unit starts its range,
// else slot G + u; the others: slot ww); a uncut unit was written whole by the
// decode kernel (to o with P == 1, to its partition state with P > 1).  The
// groups of a partition combine through LDS; with P > 1 the partition state
// goes to the documented workspace (an empty partition as (0, -inf)) and the
// partitions fold into o and lse.  With P == 1 a row whose sequence no
// boundary cuts has nothing to do.
constexpr int kMergeGroups = 8;

struct MergeState {
  float m, l, acc[4];  // base-2 reference max, sum of weights, weighted sum of o
};

// fold a normalised state (natural-log lse, o) into st
__device__ __forceinline__ void fold(MergeState& st, float lse_nat, f32x4_t v) {
  const float l2 = lse_nat * kLog2e;
  if (lse_nat == -INFINITY) return;  // an empty state drops out whatever v holds
  const float mn = fmaxf(st.m, l2);
  const float r = fast_exp2(st.m - mn);  // 0 while m is still -inf
  const float wt = fast_exp2(l2 - mn);
  st.l = st.l * r + wt;
#pragma unroll
  for (int e = 0; e < 4; ++e) st.acc[e] = st.acc[e] * r + wt * v[e];
  st.m = mn;
}

// fold another running state (base-2 max m2, sum l2, weighted sum a2)
__device__ __forceinline__ void fold_state(MergeState& st, float m2, float l2, f32x4_t a2) {
  if (m2 == -INFINITY) return;
  const float mn = fmaxf(st.m, m2);
  const float r = fast_exp2(st.m - mn);
  const float r2 = fast_exp2(m2 - mn);
  st.l = st.l * r + l2 * r2;
#pragma unroll
  for (int e = 0; e < 4; ++e) st.acc[e] = st.acc[e] * r + a2[e] * r2;
  st.m = mn;
}

__global__ __launch_bounds__(32 * kMergeGroups) void balanced_merge_kernel(BalParams p) {
  __shared__ float sm_m[kMergeGroups], sm_l[kMergeGroups];
  __shared__ f32x4_t sm_o[kMergeGroups][32];
  const int grp = threadIdx.x >> 5;
  const int lane = threadIdx.x & 31;
  const int row = blockIdx.x;
  const int b = row / p.hq;
  const int h = row - b * p.hq;
  const int P = p.num_partitions;
  const int total = p.meta[p.units];
  if (P == 1) {  // uniform over the work-group
    const int us = p.meta[b], ue = p.meta[b + 1];
    if (ue == us) return;
    const int w0 = range_of(us, total, p.G), w1 = range_of(ue - 1, total, p.G);
    if (w0 == w1) return;
    if (w1 - w0 < 8) {  // one batch of pieces: group 0 alone, no barrier
      if (grp != 0) return;
      const int first = range_start(w0, total, p.G) == us ? w0 : p.G + b;
      float lv[8];
      f32x4_t ov[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int wj = w0 + j;
        const bool ok = wj <= w1 && (wj == w0 || range_start(wj, total, p.G) <
                                                    range_start(wj + 1, total, p.G));
        const int64_t srow = (int64_t)(wj == w0 ? first : wj) * p.hq + h;
        lv[j] = ok ? p.piece_lse[srow] : -INFINITY;
        ov[j] = ok ? *reinterpret_cast<const f32x4_t*>(p.piece_o + srow * kHeadDim + 4 * lane)
                   : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      MergeState st = {-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int j = 0; j < 8; ++j) fold(st, lv[j], ov[j]);
      const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
      *reinterpret_cast<u32x2_t*>(p.o + (int64_t)row * kHeadDim + 4 * lane) =
          u32x2_t{pack_bf16x2(st.acc[0] * inv, st.acc[1] * inv),
                  pack_bf16x2(st.acc[2] * inv, st.acc[3] * inv)};
      if (lane == 0 && p.lse != nullptr)
        p.lse[row] = st.l > 0.f ? (st.m + __log2f(st.l)) * kLn2 : -INFINITY;
      return;
    }
  }
  const int gpp = P >= kMergeGroups ? 1 : kMergeGroups / P;  // groups per partition
  const int ppp = kMergeGroups / gpp;                         // partitions per pass
  const int pl = grp / gpp;  // this group's partition within the pass
  const int si = grp - pl * gpp;
  MergeState fin = {-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}};
  for (int base = 0; base < P; base += ppp) {
    const int part = base + pl;
    const bool mine = pl < ppp && part < P;
    MergeState st = {-INFINITY, 0.f, {0.f, 0.f, 0.f, 0.f}};
    bool write_state = false;  // P > 1: this partition's state is written here
    const int64_t prow = (int64_t)row * P + part;
    if (mine) {
      const int u = b * P + part;
      const int us = p.meta[u], ue = p.meta[u + 1];
      if (ue == us) {
        write_state = P > 1;
      } else {
        const int w0 = range_of(us, total, p.G);
        const int w1 = range_of(ue - 1, total, p.G);
        if (w0 == w1) {
          if (si == 0 && P > 1)
            fold(st, p.ws_lse[prow],
                 *reinterpret_cast<const f32x4_t*>(p.ws_o + prow * kHeadDim + 4 * lane));
        } else {
          write_state = P > 1;
          const int first = range_start(w0, total, p.G) == us ? w0 : p.G + u;
          // this group's pieces: w0 + si, w0 + si + gpp, ..., eight loads in flight
          for (int ww0 = w0 + si; ww0 <= w1; ww0 += 8 * gpp) {
            float lv[8];
            f32x4_t ov[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int wj = ww0 + j * gpp;
              // a range with no pages (more ranges than pages) wrote no piece
              const bool ok = wj <= w1 && (wj == w0 || range_start(wj, total, p.G) <
                                                          range_start(wj + 1, total, p.G));
              const int64_t srow = (int64_t)(wj == w0 ? first : wj) * p.hq + h;
              lv[j] = ok ? p.piece_lse[srow] : -INFINITY;
              ov[j] = ok ? *reinterpret_cast<const f32x4_t*>(p.piece_o + srow * kHeadDim +
                                                              4 * lane)
                         : f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) fold(st, lv[j], ov[j]);
          }
        }
      }
    }
    // the groups of a partition combine into its first group
    if (lane == 0) {
      sm_m[grp] = st.m;
      sm_l[grp] = st.l;
    }
    sm_o[grp][lane] = f32x4_t{st.acc[0], st.acc[1], st.acc[2], st.acc[3]};
    __syncthreads();
    if (mine && si == 0) {
      for (int k = 1; k < gpp; ++k)
        fold_state(st, sm_m[grp + k], sm_l[grp + k], sm_o[grp + k][lane]);
      if (write_state) {
        const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
        *reinterpret_cast<f32x4_t*>(p.ws_o + prow * kHeadDim + 4 * lane) =
            f32x4_t{st.acc[0] * inv, st.acc[1] * inv, st.acc[2] * inv, st.acc[3] * inv};
        if (lane == 0) p.ws_lse[prow] = st.l > 0.f ? (st.m + __log2f(st.l)) * kLn2 : -INFINITY;
      }
    }
    __syncthreads();
    // the partitions of the pass fold into group 0's running state
    if (mine && si == 0) {
      if (lane == 0) {
        sm_m[pl] = st.m;
        sm_l[pl] = st.l;
      }
      sm_o[pl][lane] = f32x4_t{st.acc[0], st.acc[1], st.acc[2], st.acc[3]};
    }
    __syncthreads();
    if (grp == 0)
      for (int k = 0; k < ppp && base + k < P; ++k) fold_state(fin, sm_m[k], sm_l[k], sm_o[k][lane]);
    __syncthreads();
  }
  if (grp != 0) return;
  const float inv = fin.l > 0.f ? 1.f / fin.l : 0.f;
  *reinterpret_cast<u32x2_t*>(p.o + (int64_t)row * kHeadDim + 4 * lane) =
      u32x2_t{pack_bf16x2(fin.acc[0] * inv, fin.acc[1] * inv),
              pack_bf16x2(fin.acc[2] * inv, fin.acc[3] * inv)};
  if (lane == 0 && p.lse != nullptr)
    p.lse[row] = fin.l > 0.f ? (fin.m + __log2f(fin.l)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_paged_decode_balanced(const DecodeLaunch& a, const BalancedLayout& ws,
                                        int G, hipStream_t stream) {
  BalParams p;
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
  p.meta = ws.meta;
  p.piece_o = ws.piece_o;
  p.piece_lse = ws.piece_lse;
  p.batch = a.batch;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.group = a.hq / a.hkv;
  p.head_tiles = (p.group + kHT - 1) / kHT;
  const int ns = p.head_tiles == 1 ? 1 : 2;  // streams per set
  p.sets_per_head = (p.head_tiles + ns - 1) / ns;
  p.total_sets = a.hkv * p.sets_per_head;
  p.nsg = (p.total_sets + kSets - 1) / kSets;
  p.num_pages = a.num_pages;
  p.num_page_entries = a.num_page_entries;
  p.max_seq_len = a.max_seq_len;
  p.num_partitions = a.num_partitions;
  p.chunk_pages = a.chunk_pages;
  p.units = a.batch * a.num_partitions;
  p.G = G;
  p.scale_log2 = a.sm_scale * kLog2e;
  // K/V loads carry the non-temporal hint (a template argument: a run-time
  // choice between the two loads would be merged into one plain load) when
  // one set reads each kv head, so every K/V row is read once
  // When every work-group holds 8 sets, each wave owns one and the waves run
  // independently (no merge between them at piece ends).
#define OXA_BAL_KERNELS(L, S)                                                   \
  {{balanced_decode_kernel<L, S, false, false>, balanced_decode_kernel<L, S, false, true>}, \
   {balanced_decode_kernel<L, S, true, false>, balanced_decode_kernel<L, S, true, true>}}
  void (*const kernels[2][2][2][2])(BalParams) = {
      {OXA_BAL_KERNELS(0, 1), OXA_BAL_KERNELS(0, 2)},
      {OXA_BAL_KERNELS(1, 1), OXA_BAL_KERNELS(1, 2)}};
#undef OXA_BAL_KERNELS
  const bool indep = p.total_sets % kSets == 0;
  void (*kernel)(BalParams) =
      kernels[a.layout == 0 ? 0 : 1][ns - 1][p.sets_per_head == 1 ? 1 : 0][indep ? 1 : 0];
  hipError_t e = launch_kernel(kernel, dim3((unsigned)(G * p.nsg)), dim3(kNW * 64),
                               (size_t)kLdsBytes, stream, p);
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.batch * a.hq;
  return launch_kernel(balanced_merge_kernel, dim3((unsigned)rows), dim3(32 * kMergeGroups), 0,
                       stream, p);
}

}  // namespace oxa
