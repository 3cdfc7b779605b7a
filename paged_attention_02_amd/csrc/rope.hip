// Standalone NeoX RoPE on q and k at explicit positions (gfx950).
//
// Operator contract: "FlashInfer parity matrix", section "Admitted attention
// matrix" (row Standard RoPE: head dim 128, NeoX split-half pairs (i, i + 64),
// explicit int32 positions) and section "Domain coverage" (RoPE: the standard
// and the Llama 3.1 variants); "Oxide Infer" README, section "Operator
// surface" (BF16 NeoX RoPE with explicit positions).  The frequency table
// arrives from the host in double precision, so one kernel serves both
// variants; angles, the rotation and the rounding to bf16 give the fused
// RoPE + append kernel's results (double-precision angles; each element the
// double rotation rounded once to bf16), the rotation formed in f32 where that
// provably gives the same bf16 (rotate_chunk_f32: 4 % faster here, 1 % slower
// in the append writer, which keeps the double form).
//
// The op is bound by HBM: every q and k row is read once and written once.
// Beyond that a token costs 64 double-precision sincos (one per lane of the
// wave that owns it, shared through LDS) and a few f32 operations per element.
// Lane l rotates frequency chunk f = l % 8 (pairs 8f .. 8f+7) of rows l / 8,
// l / 8 + 8, ... of the token, q heads first, then k heads, and issues the
// loads of four such rows before rotating any of them.
#include "device_common.h"
#include "kernels.h"

namespace oxa {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsInFlight = 4;
constexpr int kMaxGroups = 16384;

struct RopeParams {
  const uint16_t* q_in;
  uint16_t* q_out;
  const uint16_t* k_in;
  uint16_t* k_out;
  const int32_t* positions;
  int32_t hq, hkv, nnz;
  double inv_freq[64];
};

__global__ __launch_bounds__(kWaves * 64) void rope_kernel(RopeParams p) {
  __shared__ double cs[kWaves][64][2];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int f = lane & 7;
  const int hsub = lane >> 3;
  const int rows = p.hq + p.hkv;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t < p.nnz;
       t += (int64_t)gridDim.x * kWaves) {
    const int pos = p.positions[t];
    {
      double sl, cl;
      sincos((double)pos * p.inv_freq[lane], &sl, &cl);
      cs[wave][lane][0] = cl;
      cs[wave][lane][1] = sl;
    }
    __builtin_amdgcn_wave_barrier();
    // f32 cos / sin of this lane's 8 frequencies; the doubles stay in LDS for
    // the rare output that needs them (the slot is rewritten only for the
    // wave's next token)
    const double(*csf)[2] = &cs[wave][8 * f];
    float cf[8], sf[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      cf[i] = (float)csf[i][0];
      sf[i] = (float)csf[i][1];
    }

    for (int r0 = hsub; r0 < rows; r0 += 8 * kRowsInFlight) {
      u32x4_t w1[kRowsInFlight], w2[kRowsInFlight];
#pragma unroll
      for (int j = 0; j < kRowsInFlight; ++j) {
        const int r = r0 + 8 * j;
        if (r < rows) {
          const uint16_t* src = r < p.hq ? p.q_in + (t * p.hq + r) * kHeadDim
                                         : p.k_in + (t * p.hkv + (r - p.hq)) * kHeadDim;
          w1[j] = ldg16_nt(src + 8 * f);
          w2[j] = ldg16_nt(src + 64 + 8 * f);
        }
      }
#pragma unroll
      for (int j = 0; j < kRowsInFlight; ++j) {
        const int r = r0 + 8 * j;
        if (r < rows) {
          uint16_t* dst = r < p.hq ? p.q_out + (t * p.hq + r) * kHeadDim
                                   : p.k_out + (t * p.hkv + (r - p.hq)) * kHeadDim;
          u32x4_t o1, o2;
          rotate_chunk_f32(w1[j], w2[j], csf, cf, sf, &o1, &o2);
          *reinterpret_cast<u32x4_t*>(dst + 8 * f) = o1;
          *reinterpret_cast<u32x4_t*>(dst + 64 + 8 * f) = o2;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_rope(const RopeLaunch& a, hipStream_t stream) {
  if (a.nnz == 0) return hipSuccess;
  RopeParams p;
  p.q_in = a.q_in;
  p.q_out = a.q_out;
  p.k_in = a.k_in;
  p.k_out = a.k_out;
  p.positions = a.positions;
  p.hq = a.q_in != nullptr ? a.hq : 0;
  p.hkv = a.k_in != nullptr ? a.hkv : 0;
  p.nnz = a.nnz;
  for (int i = 0; i < 64; ++i) p.inv_freq[i] = a.inv_freq[i];
  int64_t groups = ((int64_t)a.nnz + kWaves - 1) / kWaves;
  if (groups > kMaxGroups) groups = kMaxGroups;
  return launch_kernel(rope_kernel, dim3((unsigned)groups), dim3(kWaves * 64), 0, stream, p);
}

}  // namespace oxa
