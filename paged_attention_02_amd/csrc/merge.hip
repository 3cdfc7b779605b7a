// Attention-state merge on gfx950.
//
// Operator: "FlashInfer parity matrix", section "Domain coverage" (Attention
// state and cascade: the state merge) and the merge step of the Single decode
// split-K row of the "Admitted attention matrix".  The state of one (row,
// head) over a key set is its softmax attention output v and the natural-log
// log-sum-exp of its scaled scores; the states of disjoint key sets combine
// into the state of their union:
//     lse = ln sum_s exp(lse_s),   v = sum_s exp(lse_s - lse) * v_s.
// A state with lse = -inf (no keys) drops out whatever its v holds; if all
// states are empty the result is (0, -inf).
//
// The merge reads every state once and does a few flops per byte: it is
// bound by HBM bandwidth (or, when small, by load latency).  Lanes own 16-byte
// pieces of the 128-wide rows (16 lanes per bf16 row, 32 per f32 row), so each
// wave reads whole rows with 16-byte loads.  A lane issues the loads of a
// batch of states together - sixteen when a unit merges more than eight (the
// split-K decode's partitions: one memory round trip instead of two), else
// eight - then folds them into a running (max, sum, accumulator) in base 2.  States are addressed through element strides, which covers both the
// operator's [row][state][head][128] layout and the split-K decode workspace
// [sequence][head][partition][128].
#include "device_common.h"
#include "kernels.h"

namespace oxa {
namespace {

constexpr int kThreads = 128;

template <bool F32>
__device__ __forceinline__ void unpack(u32x4_t w, float* x) {
  if constexpr (F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  }
}

// KB: states whose loads are in flight together
template <bool IN_F32, bool OUT_F32, bool PAIR, int KB>
__global__ __launch_bounds__(kThreads) void merge_states_kernel(MergeLaunch p) {
  constexpr int kEsz = IN_F32 ? 4 : 2;    // bytes per input element
  constexpr int kEpl = 16 / kEsz;         // elements per lane
  constexpr int kLpu = kHeadDim / kEpl;   // lanes per (row, head)
  constexpr int kUpb = kThreads / kLpu;   // (row, head) units per work-group
  const int tid = threadIdx.x;
  const int64_t unit = (int64_t)blockIdx.x * kUpb + tid / kLpu;
  if (unit >= p.units) return;
  const int piece = tid % kLpu;
  const int64_t row = unit / p.heads;
  const int64_t h = unit - row * p.heads;
  const int64_t voff = row * p.v_row + h * p.v_head + (int64_t)piece * kEpl;
  const int64_t loff = row * p.l_row + h * p.l_head;
  const unsigned char* v0 = static_cast<const unsigned char*>(p.v[0]);
  const unsigned char* v1 = static_cast<const unsigned char*>(p.v[1]);

  constexpr int kB = PAIR ? 2 : KB;
  float m = -INFINITY, wsum = 0.f, acc[kEpl];
#pragma unroll
  for (int e = 0; e < kEpl; ++e) acc[e] = 0.f;

  for (int s0 = 0; s0 < p.states; s0 += kB) {
    float l[kB];
    u32x4_t w[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      // past the last state, re-read the last one (always in bounds, so the
      // loads need no branch) and mark it empty
      const bool in = s0 + j < p.states;
      const int s = in ? s0 + j : p.states - 1;
      const float* lp;
      const unsigned char* vp;
      if (PAIR) {
        lp = (s == 0 ? p.lse[0] : p.lse[1]) + loff;
        vp = (s == 0 ? v0 : v1) + voff * kEsz;
      } else {
        lp = p.lse[0] + loff + (int64_t)s * p.l_state;
        vp = v0 + (voff + (int64_t)s * p.v_state) * kEsz;
      }
      const float lv = *lp;
      l[j] = in ? lv * kLog2e : -INFINITY;
      w[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vp));
    }
    // every load of the batch is issued before any is used: one memory round
    // trip per batch (the compiler otherwise waits for the lse values first
    // and streams the rows in a few at a time)
    __builtin_amdgcn_sched_group_barrier(0x020, 2 * kB, 0);
    __builtin_amdgcn_sched_barrier(0);
    float cm = m;
#pragma unroll
    for (int j = 0; j < kB; ++j) cm = fmaxf(cm, l[j]);
    // no branch on "nothing live yet": with every lse so far -inf, the
    // reference is 0, every weight exp2(-inf) = 0, and the state stays empty
    const float cref = cm == -INFINITY ? 0.f : cm;
    const float r = fast_exp2(m - cref);  // 0 while m is still -inf
    wsum *= r;
#pragma unroll
    for (int e = 0; e < kEpl; ++e) acc[e] *= r;
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      float x[kEpl];
      unpack<IN_F32>(w[j], x);
      const float wt = fast_exp2(l[j] - cref);  // 0 for an empty state
      const bool live = l[j] != -INFINITY;
      wsum += wt;
#pragma unroll
      for (int e = 0; e < kEpl; ++e) acc[e] = live ? fmaf(wt, x[e], acc[e]) : acc[e];
    }
    m = cm;
  }

  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if constexpr (OUT_F32) {
    float* out = static_cast<float*>(p.out) + unit * kHeadDim + piece * kEpl;
#pragma unroll
    for (int e = 0; e < kEpl; e += 4) {
      const u32x4_t o4 = {__float_as_uint(acc[e] * inv), __float_as_uint(acc[e + 1] * inv),
                          __float_as_uint(acc[e + 2] * inv), __float_as_uint(acc[e + 3] * inv)};
      *reinterpret_cast<u32x4_t*>(out + e) = o4;
    }
  } else {
    uint16_t* out = static_cast<uint16_t*>(p.out) + unit * kHeadDim + piece * kEpl;
    if constexpr (kEpl == 8) {
      const u32x4_t o4 = {pack_bf16x2(acc[0] * inv, acc[1] * inv),
                          pack_bf16x2(acc[2] * inv, acc[3] * inv),
                          pack_bf16x2(acc[4] * inv, acc[5] * inv),
                          pack_bf16x2(acc[6] * inv, acc[7] * inv)};
      *reinterpret_cast<u32x4_t*>(out) = o4;
    } else {
      const u32x2_t o2 = {pack_bf16x2(acc[0] * inv, acc[1] * inv),
                          pack_bf16x2(acc[2] * inv, acc[3] * inv)};
      *reinterpret_cast<u32x2_t*>(out) = o2;
    }
  }
  if (piece == 0 && p.lse_out != nullptr)
    p.lse_out[unit] = wsum > 0.f ? (m + __log2f(wsum)) * kLn2 : -INFINITY;
}

template <bool IN_F32, bool OUT_F32>
hipError_t launch_t(const MergeLaunch& a, hipStream_t stream) {
  constexpr int kUpb = kThreads / (kHeadDim / (16 / (IN_F32 ? 4 : 2)));
  const int64_t groups = (a.units + kUpb - 1) / kUpb;
  void (*kernel)(MergeLaunch) = a.pair         ? merge_states_kernel<IN_F32, OUT_F32, true, 2>
                                : a.states > 8 ? merge_states_kernel<IN_F32, OUT_F32, false, 16>
                                               : merge_states_kernel<IN_F32, OUT_F32, false, 8>;
  return launch_kernel(kernel, dim3((unsigned)groups), dim3(kThreads), 0, stream, a);
}

}  // namespace

int64_t merge_states_groups(int64_t units, int in_f32) {
  const int64_t upb = kThreads / (kHeadDim / (in_f32 ? 4 : 8));
  return (units + upb - 1) / upb;
}

hipError_t launch_merge_states(const MergeLaunch& a, hipStream_t stream) {
  if (a.units == 0) return hipSuccess;
  if (a.in_f32)
    return a.out_f32 ? launch_t<true, true>(a, stream) : launch_t<true, false>(a, stream);
  return a.out_f32 ? launch_t<false, true>(a, stream) : launch_t<false, false>(a, stream);
}

}  // namespace oxa
