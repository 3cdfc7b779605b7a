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
// (partition, kv head, tile of up to 16 grouped q heads, sequence), four
// waves each.  A group of more than 16 q heads is served by several
// work-groups that read the same K/V; they are placed on the same XCD (work
// groups are handed to the 8 XCDs round-robin by linear id), where the two
// reads of a row mostly meet in L2.  Each wave walks 32-token
// blocks (two pages) of the partition with its own online-softmax state; the
// waves merge through LDS at the end.
//
// Per block a wave loads K and V rows with whole-cache-line non-temporal loads
// (16 lanes per 256-byte row; the hint keeps streamed rows from displacing
// reusable lines, and after a large write a plain load of them is twice as
// slow), into registers while the previous block is computed from LDS, then
// stages them into its LDS slice (XOR-swizzled rows).  S^T = K Q^T
// takes 8 v_mfma_f32_16x16x32_bf16 (tokens are M, the q heads N); each lane
// then holds one head and 8 tokens, so the softmax max is an in-register
// reduction plus two lane exchanges, and the probabilities already form the
// B operand of O^T = V^T P^T (8 more MFMAs, V^T through the LDS transpose
// read).
#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace oxa {
namespace {

constexpr int kStatusPageRange = 16;
constexpr int kStatusIndptr = 17;
constexpr int kStatusSeqLen = 18;

constexpr int kNW = 4;                 // waves per work-group
constexpr int kHT = 16;                // q heads per work-group (MFMA N)
constexpr int kPidWin = 1024;          // page ids of a partition staged in LDS per window
constexpr int kStageBytes = 32 * 256;  // one 32-token block of K (or V) rows

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
  int32_t num_items;  // batch * hkv * num_partitions
  float scale_log2;
};

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// LDS byte offset of 16-byte chunk `c` of row `row` in a tile of 256-byte rows,
// chunks XOR-swizzled by 2*(row % 8) + (row / 8) % 2.  Conflict-free for the
// three access patterns used here: 16 lanes writing one row's 16 chunks;
// 16 lanes reading one chunk of 16 consecutive rows (the K operand); and the
// 16x16x32 transpose read, where 32 lanes read 8 consecutive rows x 32 bytes.
__device__ __forceinline__ int swz16(int row, int c) {
  const int sw = ((row & 7) << 1) | ((row >> 3) & 1);
  return row * 256 + ((c ^ sw) << 4);
}


struct BlockLoad {
  u32x4_t k[8];
  u32x4_t v[8];
};

template <int LAYOUT>
__global__ __launch_bounds__(kNW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void paged_decode_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  // Work-group -> work item.  Linear ids go to XCDs round-robin (id % 8), so
  // the head tiles of one (partition, sequence, kv head) share an XCD.
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int rest = id >> 3;
  const int ht = rest % p.head_tiles;
  const int item = (rest / p.head_tiles) * 8 + xcd;
  if (item >= p.num_items) return;  // padding of the XCD mapping
  // Items are numbered (partition, sequence, kv head) with the partition
  // slowest, so each XCD receives an even share of every partition index
  // (later partitions of short sequences are empty).
  const int kvh = item % p.hkv;
  const int b = (item / p.hkv) % p.batch;
  const int part = item / (p.hkv * p.batch);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;  // MFMA N index: q head within the tile
  const int gq = lane >> 4;   // which quarter of the k slots this lane holds

  // ---- sequence metadata (uniform) --------------------------------------
  const int L = p.seq_lens[b];
  const int lo = p.page_indptr[b];
  const int hi = p.page_indptr[b + 1];
  const bool len_ok = L >= 1 && L <= p.max_seq_len;
  const bool ptr_ok = lo >= 0 && hi >= lo && hi <= p.num_page_entries &&
                      (int64_t)(hi - lo) * kPage >= (int64_t)L;
  const bool seq_ok = len_ok && ptr_ok;

  const int chunk_tokens = p.chunk_pages * kPage;
  const int t0 = part * chunk_tokens;
  const int t1 = seq_ok ? min(t0 + chunk_tokens, L) : t0;
  const int npages = t1 > t0 ? (t1 - t0 + kPage - 1) / kPage : 0;

  // ---- Q^T fragments (B operand), loaded once: lane l holds head l%16,
  // dims 32*kk + 8*(l/16) .. +8 for k-step kk
  const int ncol = min(kHT, p.group - ht * kHT);  // real q heads in this tile
  const bool col_ok = col < ncol;
  const int head = kvh * p.group + ht * kHT + col;
  u32x4_t qf[4];
  if (col_ok) {
    const uint16_t* qp = p.q + ((int64_t)b * p.hq + head) * kHeadDim + 8 * gq;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = ldg16(qp + 32 * kk);
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = u32x4_t{0, 0, 0, 0};
  }

  f32x4_t acc[8];  // O^T: d-block j holds dims 16j + 4*(l/16) + i for head l%16
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;

  int* pids = reinterpret_cast<int*>(smem);                         // [kPidWin]
  unsigned char* ks = smem + kPidWin * 4 + wave * 2 * kStageBytes;  // K rows
  unsigned char* vs = ks + kStageBytes;                             // V rows
  const int i16 = lane & 15;
  const uint16_t* kbase = p.kp + (int64_t)kvh * (LAYOUT == 0 ? kHeadDim : kPage * kHeadDim);
  const uint16_t* vbase = p.vp + (int64_t)kvh * (LAYOUT == 0 ? kHeadDim : kPage * kHeadDim);
  // elements between consecutive slots of one kv head inside a page
  const int row_stride = LAYOUT == 0 ? p.hkv * kHeadDim : kHeadDim;
  const int64_t page_elems = (int64_t)kPage * p.hkv * kHeadDim;
  const int64_t lane_off = (int64_t)(lane >> 4) * row_stride + 8 * (lane & 15);

  for (int w0 = 0; w0 < npages; w0 += kPidWin) {
    const int wpages = min(kPidWin, npages - w0);
    __syncthreads();
    for (int i = tid; i < ((wpages + 1) & ~1); i += kNW * 64) {  // even count: blocks read pairs
      const int pid = i < wpages ? p.page_indices[lo + t0 / kPage + w0 + i] : -1;
      pids[i] = (pid >= 0 && pid < p.num_pages) ? pid : -1;
    }
    __syncthreads();
    const int tw = t0 + w0 * kPage;                 // first token of the window
    const int tw1 = min(t1, tw + kPidWin * kPage);  // end of the window
    const int nb = (tw1 - tw + 31) / 32;

    // Issue the K/V loads of window block `blk`: load s brings rows 4s .. 4s+3
    // of the 32-token block, 16 lanes per 256-byte row.  Unconditional loads
    // (straight-line code keeps the wait counters exact): a missing or invalid
    // page reads page 0 and those rows are discarded; a block past the
    // window's end re-reads its last block (a cache hit, never used).
    // The page-id pair of block blk (pair of a block past the window's end:
    // its last block's).
    auto pair_of = [&](int blk) {
      const int bi = min(blk, nb - 1);
      return int2{max(pids[2 * bi], 0), max(pids[2 * bi + 1], 0)};
    };
    auto issue = [&](int2 pp, BlockLoad& bl) {
      const int pa = __builtin_amdgcn_readfirstlane(pp.x);
      const int pb = __builtin_amdgcn_readfirstlane(pp.y);
      const uint16_t* ka = kbase + pa * page_elems + lane_off;
      const uint16_t* kb = kbase + pb * page_elems + lane_off;
      const uint16_t* va = vbase + pa * page_elems + lane_off;
      const uint16_t* vb = vbase + pb * page_elems + lane_off;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bl.k[s] = ldg16_nt(ka + 4 * s * row_stride);
        bl.v[s] = ldg16_nt(va + 4 * s * row_stride);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bl.k[4 + s] = ldg16_nt(kb + 4 * s * row_stride);
        bl.v[4 + s] = ldg16_nt(vb + 4 * s * row_stride);
      }
    };

    // Write a loaded block into this wave's LDS rows; V rows of tokens that
    // do not exist become zeros (their K rows are masked in `compute`).
    auto stage = [&](int blk, const BlockLoad& bl) {
      const int tb = tw + blk * 32;
      const bool okA = pids[2 * blk] >= 0;
      const bool okB = (tb + kPage < tw1) && pids[2 * blk + 1] >= 0;
      const bool full = (tb + 32 <= tw1) && okA && okB;  // wave-uniform
#pragma unroll
      for (int st = 0; st < 8; ++st)
        *reinterpret_cast<u32x4_t*>(ks + swz16(4 * st + (lane >> 4), lane & 15)) = bl.k[st];
      if (full) {
#pragma unroll
        for (int st = 0; st < 8; ++st)
          *reinterpret_cast<u32x4_t*>(vs + swz16(4 * st + (lane >> 4), lane & 15)) = bl.v[st];
      } else {
        // a bit mask, not a select: a select of the 16-byte rows is turned
        // into a branch per row
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int r = 4 * st + (lane >> 4);
          const uint32_t m = ((tb + r < tw1) && (st < 4 ? okA : okB)) ? 0xffffffffu : 0u;
          const u32x4_t v = bl.v[st];
          *reinterpret_cast<u32x4_t*>(vs + swz16(r, lane & 15)) =
              u32x4_t{v[0] & m, v[1] & m, v[2] & m, v[3] & m};
        }
      }
    };

    // Attention over the block staged in LDS.
    auto compute = [&](int blk) {
      const int tb = tw + blk * 32;
      const bool okA = pids[2 * blk] >= 0;
      const bool okB = (tb + kPage < tw1) && pids[2 * blk + 1] >= 0;
      const bool full = (tb + 32 <= tw1) && okA && okB;  // wave-uniform
      // S^T[token][head] for tokens 16*mb .. +15: A operand of lane l is row
      // 16*mb + l%16, dims 32*kk + 8*(l/16) .. +8
      f32x4_t s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          s[mb] = mfma_16x16x32(
              *reinterpret_cast<const u32x4_t*>(ks + swz16(16 * mb + i16, 4 * kk + gq)), qf[kk],
              s[mb]);
      }
      // this lane's tokens: 16*mb + 4*gq + i; raw-score max (scale >= 0)
      float mraw = -INFINITY;
      if (full) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mraw = fmaxf(mraw, s[mb][i]);
      } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 16 * mb + 4 * gq + i;
            const bool ok = (tb + t < tw1) && (mb == 0 ? okA : okB);
            s[mb][i] = ok ? s[mb][i] : -INFINITY;
            mraw = fmaxf(mraw, s[mb][i]);
          }
      }
      // a block with no visible key keeps max -inf (also for a zero scale,
      // where -inf * 0 would be NaN)
      const float mred = pair_max32(pair_max16(mraw));
      const float mblk = mred == -INFINITY ? -INFINITY : mred * p.scale_log2;
      // Lazy rescaling: exponentials are taken against a reference max that
      // only moves when a score exceeds it by more than 2^8, so probabilities
      // stay <= 256 and the accumulator is rescaled rarely.  The result is
      // the same softmax (the reference cancels in o = acc / l).
      if (__builtin_amdgcn_ballot_w64(mblk > m + 8.f) != 0) {
        const float mnew = mblk > m + 8.f ? mblk : m;
        const float corr = fast_exp2(m - mnew);  // 0 while m is still -inf
        lsum *= corr;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= corr;
        m = mnew;
      }
      const float muse = m == -INFINITY ? 0.f : m;
      float pv[8];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[4 * mb + i] = fast_exp2(fmaf(s[mb][i], p.scale_log2, -muse));
      if (!full) {
        // masked keys weigh exactly 0: with a zero scale fmaf(-inf, 0, x) is
        // NaN, so the weight is selected, not computed
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = s[i >> 2][i & 3] == -INFINITY ? 0.f : pv[i];
      }
      lsum += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
      // P^T B operand: k slot j of lane l is token (j < 4 ? 4gq + j : 16 + 4gq + j - 4)
      const u32x4_t pf = u32x4_t{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]),
                                 pack_bf16x2(pv[4], pv[5]), pack_bf16x2(pv[6], pv[7])};
      // O^T[d][head] += V^T[d][token] P^T[token][head] for 8 d-blocks of 16;
      // V^T through the transpose read: lanes 4e..4e+3 of each 16-lane group
      // address row (4*gq + e) (then 16 + ...) and 16 dims of d-block j
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = 2 * j + ((i16 & 3) >> 1);
        const int b8 = 8 * (i16 & 1);
        const int r = 4 * gq + (i16 >> 2);
        const u32x2_t a0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(vs + swz16(r, c) + b8));
        const u32x2_t a1 = lds_read_tr16(reinterpret_cast<const uint16_t*>(vs + swz16(r + 16, c) + b8));
        acc[j] = mfma_16x16x32(u32x4_t{a0[0], a0[1], a1[0], a1[1]}, pf, acc[j]);
      }
    };

    // One register set holds the next block's loads while the current one is
    // computed from LDS; the loaded block is staged at the end of the step.
    // The page ids of the next issue are read a step ahead, before this
    // step's LDS writes, so the loads go out as soon as the staged block is
    // written instead of after an LDS read queued behind those writes.
    BlockLoad bl;
    int blk = wave;
    int2 pp = pair_of(blk);
    if (blk < nb) {
      issue(pp, bl);
      pp = pair_of(blk + kNW);
      stage(blk, bl);
    }
    while (blk < nb) {
      const int nxt = blk + kNW;
      issue(pp, bl);
      pp = pair_of(nxt + kNW);
      compute(blk);
      if (nxt < nb) stage(nxt, bl);
      blk = nxt;
    }
  }

  // ---- merge the waves' states through LDS -------------------------------
  lsum = pair_sum32(pair_sum16(lsum));
  __syncthreads();  // staging area is reused below
  float* red_m = reinterpret_cast<float*>(smem);  // [kNW][16]
  float* red_l = red_m + kNW * kHT;               // [kNW][16]
  float* col_m = red_l + kNW * kHT;               // [16]
  float* col_l = col_m + kHT;                     // [16]
  float* red_o = col_l + kHT;                     // [kNW][128][16]
  if (gq == 0) {
    red_m[wave * kHT + col] = m;
    red_l[wave * kHT + col] = lsum;
  }
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kNW; ++w) M = fmaxf(M, red_m[w * kHT + col]);
  const float Muse = M == -INFINITY ? 0.f : M;
  float Ltot = 0.f;
#pragma unroll
  for (int w = 0; w < kNW; ++w) Ltot += red_l[w * kHT + col] * fast_exp2(red_m[w * kHT + col] - Muse);
  // this wave's share, already normalised by the total softmax sum
  const float f = Ltot > 0.f ? fast_exp2(m - Muse) / Ltot : 0.f;
  if (wave == 0 && gq == 0) {
    col_m[col] = M;
    col_l[col] = Ltot;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      red_o[(wave * kHeadDim + 16 * j + 4 * gq + i) * kHT + col] = acc[j][i] * f;
  __syncthreads();
  const bool split = p.num_partitions > 1;
  {
    // thread (c, dc): q head c of the tile, dims 8*dc .. 8*dc+7, one 16-byte store
    const int c = tid >> 4;
    const int dc = tid & 15;
    if (c < ncol) {
      float val[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) v += red_o[(w * kHeadDim + 8 * dc + i) * kHT + c];
        val[i] = v;
      }
      const float lc = col_l[c];
      const float lse_val = lc > 0.f ? (col_m[c] + __log2f(lc)) * kLn2 : -INFINITY;
      const int64_t hrow = (int64_t)b * p.hq + kvh * p.group + ht * kHT + c;
      if (split) {
        const int64_t prow = hrow * p.num_partitions + part;
        float* dst = p.ws_o + prow * kHeadDim + 8 * dc;
        *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{val[0], val[1], val[2], val[3]};
        *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{val[4], val[5], val[6], val[7]};
        if (dc == 0) p.ws_lse[prow] = lse_val;
      } else {
        *reinterpret_cast<u32x4_t*>(p.o + hrow * kHeadDim + 8 * dc) =
            u32x4_t{pack_bf16x2(val[0], val[1]), pack_bf16x2(val[2], val[3]),
                    pack_bf16x2(val[4], val[5]), pack_bf16x2(val[6], val[7])};
        if (dc == 0 && p.lse != nullptr) p.lse[hrow] = lse_val;
      }
    }
  }

  // ---- per-sequence status, after the attention so that it does not delay
  // the start of the K/V stream of the sequence's first work-group
  if (p.status != nullptr && part == 0 && kvh == 0 && ht == 0) {
    int code = 0;
    if (!len_ok) {
      code = kStatusSeqLen;
    } else if (!ptr_ok) {
      code = kStatusIndptr;
    } else {
      const int need = (L + kPage - 1) / kPage;
      int bad = 0;
      for (int i = tid; i < need; i += kNW * 64) {
        const int pid = p.page_indices[lo + i];
        bad |= (pid < 0 || pid >= p.num_pages);
      }
      if (__syncthreads_or(bad)) code = kStatusPageRange;
    }
    if (tid == 0) p.status[b] = code;
  }

}

template <int LAYOUT>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  const size_t stage = (size_t)kPidWin * 4 + (size_t)kNW * 2 * kStageBytes;
  const size_t reduce = ((size_t)kNW * 2 * kHT + 2 * kHT) * sizeof(float) +
                        (size_t)kNW * kHeadDim * kHT * sizeof(float);
  const size_t lds = stage > reduce ? stage : reduce;
  const int64_t groups = ((int64_t)(p.num_items + 7) / 8) * 8 * p.head_tiles;
  return launch_kernel(paged_decode_kernel<LAYOUT>, dim3((unsigned)groups), dim3(kNW * 64), lds,
                       stream, p);
}

}  // namespace

// Scratch of the allocation-free decode entry point: the split-K partial
// states (o_part, then lse_part) of one call live here instead of in a
// caller workspace.  Each GPU holds its own copy for the life of the process;
// every call on that GPU reuses it (a call writes every partial state it
// later reads, so nothing needs clearing), and calls that overlap on one GPU
// race on it.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch_address(void** ptr) {
  // The array's name is a host-side stand-in; its device address is resolved
  // once per device, with that device current, and kept.
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

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
  p.head_tiles = (p.group + kHT - 1) / kHT;
  p.num_pages = a.num_pages;
  p.num_page_entries = a.num_page_entries;
  p.max_seq_len = a.max_seq_len;
  p.num_partitions = a.num_partitions;
  p.chunk_pages = a.chunk_pages;
  p.num_items = a.batch * a.hkv * a.num_partitions;
  p.scale_log2 = a.sm_scale * kLog2e;
  hipError_t e = a.layout == 0 ? launch_decode_t<0>(p, stream) : launch_decode_t<1>(p, stream);
  if (e != hipSuccess || a.num_partitions == 1) return e;
  // merge the partitions: workspace [batch][hq][P][128] f32 -> o bf16
  MergeLaunch m = {};
  m.v[0] = a.ws_o;
  m.lse[0] = a.ws_lse;
  m.v_row = (int64_t)a.hq * a.num_partitions * kHeadDim;
  m.v_head = (int64_t)a.num_partitions * kHeadDim;
  m.v_state = kHeadDim;
  m.l_row = (int64_t)a.hq * a.num_partitions;
  m.l_head = a.num_partitions;
  m.l_state = 1;
  m.units = (int64_t)a.batch * a.hq;
  m.heads = a.hq;
  m.states = a.num_partitions;
  m.in_f32 = 1;
  m.out_f32 = 0;
  m.pair = 0;
  m.out = a.o;
  m.lse_out = a.lse;
  return launch_merge_states(m, stream);
}

}  // namespace oxa
