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
// Eight waves (two per SIMD) take 32 columns each.  Per 64-key tile a wave
// forms S^T = K * Q^T (16 x v_mfma_f32_32x32x16_bf16, K from LDS, Q^T resident
// in registers), masks only where the tile crosses the causal diagonal or the
// sequence end, updates the f32 online softmax (lazy rescaling), and
// accumulates O^T = V^T * P^T (16 more MFMAs; V^T through the LDS transpose
// read, P^T straight from the score registers).  K/V tiles are double-buffered
// in LDS: the next tile streams from memory straight into the other buffer (no
// register staging) during the current tile's math.  The grid is persistent
// (one work-group per CU); every work-group derives the same longest-first
// list of (sequence, query tile, kv head) items and takes its share of it.
#include <atomic>

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
constexpr int kLoadIters = kBN * 16 / (kNW * 64);  // 16-byte K (and V) loads per thread per tile
constexpr int kCols = kNW * 32;       // (row, head) columns per work-group
constexpr int kTileBytes = kBN * 256;  // one K (or V) tile: 64 rows of 256 bytes, swizzled
constexpr int kMaxLevels = 4096;       // query tiles per sequence the schedule can order

template <int N>
struct BufTag { static constexpr int value = N; };

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
  // split > 1: each item's key tiles are cut into `split` contiguous chunks
  // whose normalised states go to ws_o [split][nnz_qo][hq][128] and ws_lse
  // [split][nnz_qo][hq] (natural log) for the merge kernel
  int32_t split;
  float* ws_o;
  float* ws_lse;
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

// LDS byte address of a pointer into shared memory (wave-uniform here).
__device__ __forceinline__ uint32_t lds_addr(const unsigned char* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)(p));
}

// 16 bytes per lane from global memory straight into LDS at base + 16 * lane
// (global_load_lds_dwordx4, LDS base in M0, which the compiler loads for the
// operand).  Written as an instruction the compiler does not track: a tracked
// one makes it wait for the transfer before the next read of any LDS, which
// would serialise the load of tile kt+1 with the math on tile kt.  The kernel
// waits for its transfers itself (vmcnt) before the barrier that hands a
// buffer to its readers.
__device__ __forceinline__ void dma16(const uint16_t* g, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" :: "v"(g), "{m0}"(lds_base) : "memory");
}

// Bring K/V tile `kt` (64 keys) straight into LDS: wave w fills rows
// 8w .. 8w+7 with two 16-byte-per-lane loads for K and two for V, each lane
// writing one fixed 16-byte slot of a 4-row block.  The lane at slot `pos` of
// row r fetches the chunk that the XOR swizzle places there (chunk pos ^ sw(r)),
// so the tile lands in the swizzled layout the readers expect.  Keys past the
// sequence end re-read its last key (finite data; their scores are masked), and
// a key on an invalid page reads page 0 (the sequence's status is then non-zero
// and its rows are unspecified), so every load stays inside K and V.
template <bool PAGED, int LAYOUT>
__device__ __forceinline__ void issue_tile(const PrefillParams& p, const SeqInfo& si, int kvh,
                                           int kt, int wave, int lane, const int* pids,
                                           int wbase, unsigned char* ks, unsigned char* vs) {
#pragma unroll
  for (int u = 0; u < kLoadIters; ++u) {
    const int row = wave * (4 * kLoadIters) + 4 * u + (lane >> 4);
    const int pos = lane & 15;
    const int sw = ((row & 3) << 2) | ((row >> 2) & 3);
    const int chunk = pos ^ sw;
    const int key = min(kt * kBN + row, si.klen - 1);
    int64_t off;
    if (!PAGED) {
      off = ((int64_t)(si.kbase + key) * p.hkv + kvh) * kHeadDim;
    } else {
      const int pid = max(pids[key / kPage - wbase], 0);
      const int slot = key & (kPage - 1);
      off = LAYOUT == 0 ? (((int64_t)pid * kPage + slot) * p.hkv + kvh) * kHeadDim
                        : (((int64_t)pid * p.hkv + kvh) * kPage + slot) * kHeadDim;
    }
    off += chunk * 8;
    const int lds_off = (wave * (4 * kLoadIters) + 4 * u) * 256;
    dma16(p.k + off, lds_addr(ks + lds_off));
    dma16(p.v + off, lds_addr(vs + lds_off));
  }
}

// Query tiles of one sequence, or 0 if its metadata is invalid.
template <bool PAGED>
__device__ __forceinline__ int seq_tiles(const PrefillParams& p, int b) {
  const SeqInfo si = seq_info<PAGED>(p, b);
  return si.code == 0 ? (si.qlen + p.bm - 1) / p.bm : 0;
}

// In-place suffix sum over a[0 .. n) in LDS: a[t] <- a[t] + a[t+1] + ... .
// Each thread owns a contiguous run of entries; the sum of all later runs
// comes from a shuffle scan inside the wave plus the totals of later waves
// (tot[0 .. kNW) holds those), so no thread walks a long serial chain of LDS
// reads - the schedule is built at the start of every work-group, and on
// short inputs it would otherwise cost more than the attention itself.
__device__ __forceinline__ void lds_suffix_sum(int* a, int n, int* tot, int tid) {
  constexpr int kThreads = kNW * 64;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = min(tid * per, n), hi = min(lo + per, n);
  int sum = 0;
  for (int u = lo; u < hi; ++u) sum += a[u];
  int incl = sum;  // sum over lanes >= this one in the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_down(incl, off, 64);
    if (lane + off < 64) incl += o;
  }
  if (lane == 0) tot[wave] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int w = wave + 1; w < kNW; ++w) run += tot[w];
  __syncthreads();
  for (int u = hi - 1; u >= lo; --u) {
    run += a[u];
    a[u] = run;
  }
  __syncthreads();
}

// Persistent kernel: gridDim.x work-groups (one per CU) share a schedule of
// every (sequence, query tile, kv head, head tile) item, ordered by query-tile
// index from the last down (the longest causal tiles first) and striped over
// the work-groups.  Each group derives the same schedule from the metadata:
// a histogram of per-sequence tile counts gives, for every tile index t, how
// many sequences have a tile t and how many items precede that level.  No
// work-group is ever idle, which matters because the hardware dispatches
// groups in order and round-robin over CUs: a regular pattern of instantly
// finishing groups would pin the live ones to a fraction of the CUs.
// SPLIT selects the key-chunked form at compile time, so the unsplit kernel
// (long prefill) carries none of its registers or code.
template <bool PAGED, int LAYOUT, bool SPLIT>
__global__ __launch_bounds__(kNW * 64) void prefill_kernel(PrefillParams p) {
  const int split = SPLIT ? p.split : 1;
  __shared__ __align__(16) unsigned char smem[4 * kTileBytes];  // K0, V0, K1, V1
  __shared__ int pids[PAGED ? kPidWin : 1];
  __shared__ int lvl_cnt[kMaxLevels + 1];   // sequences with more than t tiles
  __shared__ int lvl_before[kMaxLevels + 1];  // items at tile indices above t
  __shared__ int red[kNW * 64];
  __shared__ int sel_b;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int gi = lane >> 5;
  const int g16 = (lane >> 4) & 1;
  const int i16 = lane & 15;
  const int G = gridDim.x;

  // ---- per-sequence status: this group covers sequences b = blockIdx.x mod G
  if (p.status != nullptr) {
    for (int b = blockIdx.x; b < p.batch; b += G) {
      const SeqInfo si = seq_info<PAGED>(p, b);
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
  }

  // ---- the schedule ------------------------------------------------------
  const int levels = p.num_tiles;  // <= kMaxLevels (host-checked)
  for (int t = tid; t <= levels; t += kNW * 64) lvl_cnt[t] = 0;
  __syncthreads();
  for (int b = tid; b < p.batch; b += kNW * 64) {
    const int n = min(seq_tiles<PAGED>(p, b), levels);
    if (n > 0) atomicAdd(&lvl_cnt[n], 1);  // histogram of tile counts
  }
  __syncthreads();
  lds_suffix_sum(lvl_cnt, levels + 1, red, tid);  // lvl_cnt[n] = #sequences with >= n tiles
  for (int t = tid; t <= levels; t += kNW * 64)
    lvl_before[t] = t + 1 <= levels ? lvl_cnt[t + 1] : 0;  // #sequences with tile t
  __syncthreads();
  // lvl_before[t] <- items (pairs) at levels >= t, then shift to levels > t
  lds_suffix_sum(lvl_before, levels + 1, red, tid);
  const int total_pairs = lvl_before[0];
  const int per_pair = p.hkv * p.head_tiles;
  const int64_t base_items = (int64_t)total_pairs * per_pair;
  const int64_t total_items = base_items * split;  // key chunk is the slowest index

  // Deal items to groups boustrophedon-style in units of 8 consecutive items
  // (same tile index, neighbouring kv heads): even rounds go 0 .. G-1, odd
  // rounds G-1 .. 0, so each group pairs long tiles with short ones, while an
  // item's position mod 8 - its XCD - is kept.
  const int G8 = G >= 8 ? G / 8 : 1;
  const int gsub = G >= 8 ? (int)(blockIdx.x & 7) : 0;
  const int gblk = G >= 8 ? (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int gw = G >= 8 ? 8 : G;
  for (int64_t round = 0; round * G < total_items; ++round) {
    const int64_t slot = (round & 1) ? (int64_t)(G8 - 1 - gblk) * gw + gsub : (int64_t)blockIdx.x;
    const int64_t item_all = round * G + slot;
    if (item_all >= total_items) continue;
    const int chunk = SPLIT ? (int)(item_all / base_items) : 0;
    const int64_t item = item_all - (int64_t)chunk * base_items;
    const int j = (int)(item / per_pair);
    const int kvh = (int)((item / p.head_tiles) % p.hkv);
    const int ht = (int)(item % p.head_tiles);
    // level t: the smallest t whose later levels hold at most j pairs
    int lo_t = 0, hi_t = levels - 1;
    while (lo_t < hi_t) {
      const int mid = (lo_t + hi_t) >> 1;
      if (lvl_before[mid + 1] <= j) hi_t = mid; else lo_t = mid + 1;
    }
    const int tile = lo_t;
    const int rank = j - lvl_before[tile + 1];
    // sequence: the rank-th (ascending) with more than `tile` tiles
    {
      int seen = 0;
      for (int b0 = 0; b0 < p.batch; b0 += kNW * 64) {
        const int bb = b0 + tid;
        const bool has = bb < p.batch && seq_tiles<PAGED>(p, bb) > tile;
        const uint64_t mask = __builtin_amdgcn_ballot_w64(has);
        const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
        if (lane == 0) red[wave] = __builtin_popcountll(mask);
        __syncthreads();
        int before = 0, here = 0;  // qualifying sequences before this wave / in this pass
        for (int w = 0; w < kNW; ++w) {
          before += w < wave ? red[w] : 0;
          here += red[w];
        }
        if (has && seen + before + pos == rank) sel_b = bb;
        __syncthreads();
        seen += here;
        if (seen > rank) break;
      }
      __syncthreads();
    }
    const int b = sel_b;

  SeqInfo si = seq_info<PAGED>(p, b);
  const int r0 = tile * p.bm;
  const int rows_here = min(p.bm, si.qlen - r0);
  const int offset = si.klen - si.qlen;  // bottom-right causal alignment
  const int kv_end = p.causal ? min(si.klen, r0 + rows_here + offset) : si.klen;
  const int ntiles = (kv_end + kBN - 1) / kBN;
  // this chunk's key tiles [kt0, kt1) (all of them without a split)
  const int kt0 = (int)((int64_t)chunk * ntiles / split);
  const int kt1 = (int)((int64_t)(chunk + 1) * ntiles / split);

  // this lane's column: (row, head) pair wave*32 + col
  const int pair = wave * 32 + col;
  const int prow = pair / p.gwg;
  const int head_in_group = ht * p.gwg + (pair - prow * p.gwg);
  const bool col_ok = prow < rows_here && pair < p.bm * p.gwg && head_in_group < p.group;
  const int qrow = r0 + prow;
  const int head = kvh * p.group + head_in_group;
  const int row_lim = qrow + offset;  // last visible key (causal)
  u32x4_t qf[8];
  if (col_ok) {
    const uint16_t* qp = p.q + ((int64_t)(si.q0 + qrow) * p.hq + head) * kHeadDim + gi * 64;
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = ldg16(qp + 8 * st);
  } else {
#pragma unroll
    for (int st = 0; st < 8; ++st) qf[st] = u32x4_t{0, 0, 0, 0};
  }

  f32x16_t acc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) acc[d] = f32x16_t{};
  // Online softmax state of this column: m is the reference (base 2, scaled)
  // the exponentials are taken against, negm = -m for the exponent FMA; +inf
  // until the first visible key, which forces the first update.
  float m = -INFINITY, negm = INFINITY, lsum = 0.f;
  // smallest visible-key limit among the work-group's rows: tiles past it need masks
  const int wg_min_lim = r0 + offset;

  // LDS byte offsets of this lane's fragments within one buffer (the buffer
  // and the 32-key half add compile-time offsets).  K: chunk 8*gi + st of
  // row col (the XOR swizzle depends on the row mod 16 only).  V^T: the
  // transpose-read addresses of rows 4*gi + i16/4 (a = 0) and +8 (a = 1),
  // 16-dim group d of the 32-dim block, 8-byte half i16 % 2.
  int koff[8], voff[4][2];
#pragma unroll
  for (int st = 0; st < 8; ++st) koff[st] = swz_off(col, 8 * gi + st);
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int r = 4 * gi + (i16 >> 2) + 8 * a;
      const int c = 4 * d + 2 * g16 + ((i16 & 3) >> 1);
      voff[d][a] = kTileBytes + swz_off(r, c) + 8 * (i16 & 1);
    }

  // Loads of a whole tile (every key exists): this lane's two 16-byte pieces
  // are fixed offsets from the tile's first key row (ragged) or from the page
  // that holds the wave's 8 rows (paged: rows 8*wave .. +7 lie in page
  // wave / 2 of the tile's 4), so a tile costs one page-id read per wave and
  // one 64-bit add per load.  The partial last tile takes issue_tile.
  uint32_t ld_off[kLoadIters];
#pragma unroll
  for (int u = 0; u < kLoadIters; ++u) {
    const int row = wave * (4 * kLoadIters) + 4 * u + (lane >> 4);
    const int sw = ((row & 3) << 2) | ((row >> 2) & 3);
    const int chunk = (lane & 15) ^ sw;
    const int slot = row & (kPage - 1);
    if (!PAGED)
      ld_off[u] = (uint32_t)((row * p.hkv + kvh) * kHeadDim + chunk * 8);
    else if (LAYOUT == 0)
      ld_off[u] = (uint32_t)((slot * p.hkv + kvh) * kHeadDim + chunk * 8);
    else
      ld_off[u] = (uint32_t)((kvh * kPage + slot) * kHeadDim + chunk * 8);
  }
  const int64_t page_elems = (int64_t)kPage * p.hkv * kHeadDim;
  static_assert(kLoadIters * 4 * kNW == kBN && kBN == 4 * kPage, "8 rows per wave, 4 pages per tile");

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
  int wbase = kt0 / kTilesPerWin * kPidWin;  // the page-id window of tile kt0
  auto issue = [&](int kt, unsigned char* ks, unsigned char* vs) {
    if (kt * kBN + kBN > si.klen) {
      issue_tile<PAGED, LAYOUT>(p, si, kvh, kt, wave, lane, pids, wbase, ks, vs);
      return;
    }
    int64_t base;
    if (PAGED) {
      // an invalid page reads page 0 (the sequence's status says so)
      const int pid = __builtin_amdgcn_readfirstlane(max(pids[kt * 4 + (wave >> 1) - wbase], 0));
      base = (int64_t)pid * page_elems;
    } else {
      base = (int64_t)(si.kbase + kt * kBN) * p.hkv * kHeadDim;
    }
#pragma unroll
    for (int u = 0; u < kLoadIters; ++u) {
      const int lds_off = (wave * (4 * kLoadIters) + 4 * u) * 256;
      dma16(p.k + base + ld_off[u], lds_addr(ks + lds_off));
      dma16(p.v + base + ld_off[u], lds_addr(vs + lds_off));
    }
  };
  if (PAGED) stage_pids(wbase);
  __syncthreads();

  // Tile kt0 goes to buffer 0, kt0 + 1 to buffer 1, and so on.
  if (kt1 > kt0) issue(kt0, smem, smem + kTileBytes);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // One 64-key tile from LDS buffer BUF (a compile-time constant, so every
  // fragment address is a per-lane register plus an immediate offset).
  auto tile_step = [&](int kt, auto buf_tag) {
    constexpr int BUF = decltype(buf_tag)::value;
    const unsigned char* ks = smem + BUF * 2 * kTileBytes;
    if (PAGED && kt + 1 < kt1 && (kt + 1) % kTilesPerWin == 0) {
      // the next tile starts a new page-id window (only tile kt+1 uses page
      // ids from here on, and every wave is past its reads of the old window)
      wbase = (kt + 1) / kTilesPerWin * kPidWin;
      __syncthreads();
      stage_pids(wbase);
      __syncthreads();
    }
    if (kt + 1 < kt1) {  // tile kt+1 streams into the other buffer meanwhile
      unsigned char* kn = smem + (1 - BUF) * 2 * kTileBytes;
      issue(kt + 1, kn, kn + kTileBytes);
    }

    const int key0 = kt * kBN;
    const bool need_mask = (key0 + kBN > si.klen) || (p.causal && key0 + kBN - 1 > wg_min_lim);
    // S^T[key][col] for keys 32*mb .. +31: 8 k-steps over the 128 dims, all
    // 8 K fragments read before the MFMAs (scheduling groups)
    auto scores = [&](int mb) {
      f32x16_t s = f32x16_t{};
      u32x4_t kf[8];
#pragma unroll
      for (int st = 0; st < 8; ++st)
        kf[st] = *reinterpret_cast<const u32x4_t*>(ks + mb * 8192 + koff[st]);
#pragma unroll
      for (int st = 0; st < 8; ++st) s = mfma_32x32x16(kf[st], qf[st], s);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // then MFMAs
      return s;
    };
    f32x16_t s_carry = f32x16_t{};  // the second half's scores
    // Two online-softmax steps of 32 keys per tile (keeps half the scores live).
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16_t s = mb == 0 ? scores(0) : s_carry;
      // V^T fragments of this half, read now so that their LDS latency passes
      // under the softmax (they do not depend on it).  Transpose read: lanes
      // 4e..4e+3 of a 16-lane group address row (32*mb + 16*h + 4*(l/32) + e)
      // (then +8), 16 dims of the 32-wide d block.
      u32x4_t vf[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const unsigned char* vb = ks + 32 * mb * 256 + 16 * h * 256;
          const u32x2_t a0 = lds_read_tr16(reinterpret_cast<const uint16_t*>(vb + voff[d][0]));
          const u32x2_t a1 = lds_read_tr16(reinterpret_cast<const uint16_t*>(vb + voff[d][1]));
          vf[h][d] = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
        }
      __builtin_amdgcn_sched_barrier(0);
      // Probabilities against the current reference, packed to bf16 pairs
      // (the P operand) and summed in f32; masked keys weigh exactly 0
      // (selected, not computed: with a zero scale fmaf(-inf, 0, x) is NaN).
      // The masked form is a separate instance so the common tiles carry none
      // of its selects.
      uint32_t pk[8];
      float psum;
      auto probs = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value != 0;
        psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p0 = fast_exp2(fmaf(s[r], p.scale_log2, negm));
          float p1 = fast_exp2(fmaf(s[r + 1], p.scale_log2, negm));
          if constexpr (MASKED) {
            p0 = s[r] == -INFINITY ? 0.f : p0;
            p1 = s[r + 1] == -INFINITY ? 0.f : p1;
          }
          pk[r >> 1] = pack_bf16x2(p0, p1);
          psum += p0 + p1;
        }
      };
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + mb * 32 + 8 * (r >> 2) + 4 * gi + (r & 3);
          const bool vis = (key < si.klen) & (!p.causal | (key <= row_lim));
          s[r] = vis ? s[r] : -INFINITY;
        }
        probs(BufTag<1>{});
      } else {
        probs(BufTag<0>{});
      }
      // Lazy reference: it moves only when this lane's 16 weights sum past
      // 2^8 (or are not finite: the first visible key, against m = -inf).
      // Then every column takes its exact running max (raw-score max times
      // the scale, which commutes with a scale >= 0), rescales its state and
      // recomputes.  The result is the same softmax: the reference cancels
      // in o = acc / l.
      if (__builtin_amdgcn_ballot_w64(!(psum <= 256.f)) != 0) {
        float mraw = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mraw = fmaxf(mraw, s[r]);
        const float mred = pair_max32(mraw);
        // a column with no visible key keeps -inf (also for a zero scale)
        const float mt = mred == -INFINITY ? -INFINITY : mred * p.scale_log2;
        if (mt > m) {
          const float corr = fast_exp2(m - mt);  // 0 while m is still -inf
          lsum *= corr;
#pragma unroll
          for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[d][r] *= corr;
          m = mt;
          negm = -mt;
        }
        if (need_mask)
          probs(BufTag<1>{});
        else
          probs(BufTag<0>{});
      }
      lsum += psum;
      // The second half's S MFMAs go ahead of this half's P.V MFMAs, so its
      // softmax can start while they still occupy the matrix core.
      if (mb == 0) {
        s_carry = scores(1);
        __builtin_amdgcn_sched_barrier(0);
      }
      // O^T += V^T * P^T over the 2 k-steps of 16 keys in this block.
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4_t pf = u32x4_t{pk[4 * h], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]};
#pragma unroll
        for (int d = 0; d < 4; ++d) acc[d] = mfma_32x32x16(vf[h][d], pf, acc[d]);
      }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile kt+1 has landed in LDS
    __syncthreads();
  };
  for (int kt = kt0; kt < kt1; kt += 2) {
    tile_step(kt, BufTag<0>{});
    if (kt + 1 < kt1) tile_step(kt + 1, BufTag<1>{});
  }

  const float ls = pair_sum32(lsum);
  if (col_ok) {
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    const int64_t hrow = (int64_t)(si.q0 + qrow) * p.hq + head;
    const float lse_val = ls > 0.f ? (m + __log2f(ls)) * kLn2 : -INFINITY;
    if (SPLIT) {  // this chunk's normalised state, f32
      const int64_t srow = (int64_t)chunk * p.nnz_qo * p.hq + hrow;
      float* wrow = p.ws_o + srow * kHeadDim;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const int dd = 32 * d + 8 * (r >> 2) + 4 * gi;
          const u32x4_t w = {__float_as_uint(acc[d][r] * inv), __float_as_uint(acc[d][r + 1] * inv),
                             __float_as_uint(acc[d][r + 2] * inv),
                             __float_as_uint(acc[d][r + 3] * inv)};
          *reinterpret_cast<u32x4_t*>(wrow + dd) = w;
        }
      if (gi == 0) p.ws_lse[srow] = lse_val;
    } else {
      uint16_t* orow = p.o + hrow * kHeadDim;
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
      if (gi == 0 && p.lse != nullptr) p.lse[hrow] = lse_val;
    }
  }
  __syncthreads();  // LDS (tiles, page ids, selection) is reused by the next item
  }
}

}  // namespace

// Compute units of the current device, queried once per device: the
// attribute query walks the runtime's device properties and costs more host
// time than a short prefill takes on the GPU.
hipError_t device_cu_count(int* cus) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices)
    cached[dev].store(*cus, std::memory_order_relaxed);
  return e;
}

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
  p.split = 1;  // raised below for a small call with the workspace for it
  p.ws_o = a.ws_o;
  p.ws_lse = a.ws_lse;
  // one persistent work-group per CU (a multiple of 8, so a kv head's items
  // stay on one XCD), never more than there can be items
  int cus = 0;
  hipError_t e = device_cu_count(&cus);
  if (e != hipSuccess) return e;
  const int64_t pairs_ub = ((int64_t)a.nnz_qo + p.bm - 1) / p.bm + a.batch;
  const int64_t items_ub = pairs_ub * p.hkv * p.head_tiles;
  // A call whose items would fill at most half of the CUs cuts each item's
  // keys into chunks (when the caller gave the workspace for it), so more
  // CUs work and each walks fewer key tiles in series; at most half as many
  // chunks as the longest item has key tiles.
  if (a.max_split > 1 && cus > 0) {
    int64_t split = a.max_split;
    const int64_t by_cus = cus / (items_ub > 0 ? items_ub : 1);
    const int64_t by_keys = ((int64_t)(a.max_kv_len + kBN - 1) / kBN + 1) / 2;
    if (split > by_cus) split = by_cus;
    if (split > by_keys) split = by_keys;
    p.split = split >= 2 ? (int32_t)split : 1;
  }
  int64_t groups = cus >= 8 ? (cus / 8) * 8 : (cus > 0 ? cus : 1);
  if (groups > items_ub * p.split) groups = items_ub > 0 ? items_ub * p.split : 1;
  dim3 grid((unsigned)groups);
  dim3 block(kNW * 64);
  const bool split = p.split > 1;
  void (*kernel)(PrefillParams);
  if (!a.paged)
    kernel = split ? prefill_kernel<false, 0, true> : prefill_kernel<false, 0, false>;
  else if (a.layout == 0)
    kernel = split ? prefill_kernel<true, 0, true> : prefill_kernel<true, 0, false>;
  else
    kernel = split ? prefill_kernel<true, 1, true> : prefill_kernel<true, 1, false>;
  e = launch_kernel(kernel, grid, block, 0, stream, p);
  if (e != hipSuccess || p.split == 1) return e;
  // merge the chunks: ws [split][nnz_qo][hq][128] f32 -> o [nnz_qo][hq][128] bf16
  MergeLaunch m = {};
  m.v[0] = a.ws_o;
  m.lse[0] = a.ws_lse;
  m.v_row = (int64_t)a.hq * kHeadDim;
  m.v_head = kHeadDim;
  m.v_state = (int64_t)a.nnz_qo * a.hq * kHeadDim;
  m.l_row = a.hq;
  m.l_head = 1;
  m.l_state = (int64_t)a.nnz_qo * a.hq;
  m.units = (int64_t)a.nnz_qo * a.hq;
  m.heads = a.hq;
  m.states = p.split;
  m.in_f32 = 1;
  m.out_f32 = 0;
  m.pair = 0;
  m.out = a.o;
  m.lse_out = a.lse;
  return launch_merge_states(m, stream);
}

}  // namespace oxa
