// Device-side helpers shared by the gfx950 kernels of liboxa.
//
// Matrix-core fragment layouts (gfx950, wave64), as used throughout:
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]
//     A operand: lane l holds A[m = l%32][k = 8*(l/32) + j], j = 0..7
//     B operand: lane l holds B[k = 8*(l/32) + j][n = l%32], j = 0..7
//     C result : lane l, reg r holds C[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32]
// A reduction over k does not depend on which physical k a lane slot stands
// for, as long as A and B use the same assignment; the kernels use that
// freedom to make every lane's global or LDS read one contiguous vector.
//
// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes,
// output lane i, element e (of 4 bf16) is source element i%4 of the 8 bytes
// addressed by lane 4*e + i/4 of the group.  If lanes 4e..4e+3 point at the
// four 8-byte pieces of a 16-element row segment of "row e", lane i receives
// column i of rows 0..3 - a 4x16 -> 16x4 transpose.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oxa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Launch a kernel whose one argument is a parameter struct; the launch's own
// status is returned (not a sticky error left by an earlier, unrelated call).
template <typename P>
inline hipError_t launch_kernel(void (*kernel)(P), dim3 grid, dim3 block, size_t lds,
                                hipStream_t stream, const P& params) {
  void* args[] = {const_cast<P*>(&params)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, lds, stream);
}

constexpr int kPage = 16;
constexpr int kHeadDim = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// bf16 halves of a 32-bit word -> f32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two f32 -> packed bf16x2 (hardware convert, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Round a double to bf16 (nearest, ties to even) in one step from its bits.
// The bf16 significand keeps 8 bits; subnormal results use the fixed quantum
// 2^-133; magnitudes that round past the largest finite bf16 become infinity.
__host__ __device__ __forceinline__ uint16_t bf16_from_double_rne(double x) {
  uint64_t u;
  __builtin_memcpy(&u, &x, 8);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const uint64_t a = u & 0x7fffffffffffffffull;
  if (a >= 0x7ff0000000000000ull)
    return (uint16_t)(a == 0x7ff0000000000000ull ? (sign | 0x7f80u) : 0x7fc0u);
  const int e = (int)(a >> 52);
  if (e == 0) return (uint16_t)sign;  // double zero or subnormal: far below bf16's range
  const int eb = e - 896;             // bf16 biased exponent of the same binade
  const uint64_t mant = (a & 0xfffffffffffffull) | 0x10000000000000ull;
  const int shift = eb >= 1 ? 45 : 46 - eb;
  if (shift > 54) return (uint16_t)sign;
  uint64_t q = mant >> shift;
  const uint64_t rem = mant & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  uint32_t bits;
  if (eb >= 1) {
    uint32_t E = (uint32_t)eb;
    if (q >> 8) { q >>= 1; ++E; }
    if (E >= 255) return (uint16_t)(sign | 0x7f80u);
    bits = (E << 7) | (uint32_t)(q & 0x7f);
  } else {
    bits = (uint32_t)q;  // a carry into 0x80 is the smallest normal, encoded alike
  }
  return (uint16_t)(sign | bits);
}

// 2^x on the transcendental unit (v_exp_f32; results below 2^-126 flush to
// zero, which a softmax weight may do)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Byte offset of 16-byte chunk `c` of row `row` in an LDS tile of 256-byte
// rows (128 bf16) whose chunks are XOR-swizzled by 4*(row % 4) + (row / 4) % 4.
// With this swizzle three access patterns are free of bank conflicts:
// 16 lanes writing the 16 chunks of one row, lanes reading one chunk of 16
// consecutive rows (the K operand), and the transpose read of 4 consecutive
// rows x 64 bytes (the V operand).
__device__ __forceinline__ int swz_off(int row, int c) {
  const int sw = ((row & 3) << 2) | ((row >> 2) & 3);
  return row * 256 + ((c ^ sw) << 4);
}

// max of v over the lane pair (l, l ^ 32)
__device__ __forceinline__ float pair_max32(float v) {
  const uint32_t b = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max and sum of v over the lane pair (l, l ^ 16)
__device__ __forceinline__ float pair_max16(float v) {
  const uint32_t b = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum16(float v) {
  const uint32_t b = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float pair_sum32(float v) {
  const uint32_t b = __float_as_uint(v);
  auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4_t ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// 16 bytes with the non-temporal hint, for data that one call reads once
// (streamed K/V rows): it keeps those lines from displacing reusable ones.
__device__ __forceinline__ u32x4_t ldg16_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// 8 bytes through the LDS transpose read; `p` is a generic pointer into LDS.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// ---- NeoX rotation helpers (RoPE in float64, one rounding to bf16) ----

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

// bf16 bits of f32 `r` rounded to nearest even, and whether that equals the
// rounding of every value within `e` of r: r must lie farther than e from the
// midpoint of its bf16 cell (r - mid is exact: same sign and exponent), and e
// must be under a quarter of r's bf16 ulp (below a power of two the cell
// underneath is half as wide).  Zero, subnormal and non-finite r never pass.
__device__ __forceinline__ uint32_t bf16_rne_checked(float r, float e, bool& ok) {
  const uint32_t u = __float_as_uint(r);
  const float mid = __uint_as_float((u & 0xffff0000u) | 0x8000u);
  const float binade = __uint_as_float(u & 0x7f800000u);  // 2^exponent(r)
  ok = ok && (fabsf(r - mid) > e) && (e * 512.f < binade);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
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

// rotate_chunk with the same results from f32 arithmetic where that is provably
// enough: y1 = x1 cos - x2 sin, y2 = x2 cos + x1 sin, each rounded once to bf16
// as the double-precision expression would be.  cs: the double (cos, sin) of
// the 8 frequencies (read only on the rare double-precision path, so it may
// stay in LDS); cf, sf: the same rounded to f32.
//
// The rotation is first formed in f32: with bf16 (hence exact f32) inputs and
// |cos|, |sin| <= 1 it is within 2^-22 (|x1| + |x2|) of the exact value for the
// double cos / sin (two roundings of cos / sin, one of the product, one of the
// FMA), and the double expression is within 2^-51 (|x1| + |x2|) of it.  An
// output whose f32 value lies farther than 2^-21 (|x1| + |x2|) from a bf16
// rounding boundary therefore rounds like the double one; a pair with any
// other output (about one in a thousand) is recomputed in double precision.
__device__ __forceinline__ void rotate_chunk_f32(u32x4_t w1, u32x4_t w2, const double (*cs)[2],
                                                 const float* cf, const float* sf, u32x4_t* out1,
                                                 u32x4_t* out2) {
  float x1[8], x2[8];
  unpack8(w1, x1);
  unpack8(w2, x2);
  uint32_t y1[8], y2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = x1[i], b = x2[i];
    // the bound, kept clear of the subnormal range where errors are absolute
    const float e = fmaxf((fabsf(a) + fabsf(b)) * 0x1p-21f, 0x1p-120f);
    bool ok = true;
    y1[i] = bf16_rne_checked(fmaf(a, cf[i], -(b * sf[i])), e, ok);
    y2[i] = bf16_rne_checked(fmaf(b, cf[i], a * sf[i]), e, ok);
    if (!ok) {  // per pair: a wave rarely has a lane here
      const double ad = a, bd = b, c = cs[i][0], sn = cs[i][1];
      y1[i] = bf16_rne(ad * c - bd * sn);
      y2[i] = bf16_rne(bd * c + ad * sn);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    (*out1)[i] = y1[2 * i] | (y1[2 * i + 1] << 16);
    (*out2)[i] = y2[2 * i] | (y2[2 * i + 1] << 16);
  }
}

}  // namespace oxa
