// Shared device helpers and host plumbing for libnvfp4 (gfx950 only).
//
// The E2M1 / E4M3 grids and the two-level scaling recipe are those of
// axbrief.com, "NVFP4: how NVIDIA pre-trained a 12B model on 10 trillion
// tokens", section "E2M1 format and two-level scaling".  The device code
// reaches the recipe's bits through gfx950's own conversion instructions
// (v_cvt_scalef32_pk_fp4_f32 rounds f32 to E2M1 to nearest-even with
// saturation, keeping the sign of zeros and underflows; v_cvt_pk_fp8_f32
// rounds to OCP E4M3 to nearest-even for inputs up to 464, so inputs are
// clamped to 448 first) and through a per-tensor reciprocal table whose
// exactness is established when the table is built (see build_entry).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

#ifndef __gfx950__
#if defined(__HIP_DEVICE_COMPILE__)
#error "libnvfp4 device code targets gfx950 only"
#endif
#endif

namespace nvfp4 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 16;          // values per E4M3 block scale
constexpr int kThreads = 256;       // threads per workgroup of the streaming kernels
constexpr float kGlobalDiv = 2688.0f;  // 6 (E2M1 max) * 448 (E4M3 max)

// ---------------------------------------------------------------- bf16 words
// A 32-bit word holds two bf16 values; element 2i is the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// max |x| over the two halves, as bf16 magnitude bits (order-preserving for
// non-negative finite values), kept packed.
__device__ __forceinline__ uint32_t pk_absmax(uint32_t acc, uint32_t w) {
  u16x2 a = __builtin_bit_cast(u16x2, acc);
  u16x2 b = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}
__device__ __forceinline__ uint32_t halves_max(uint32_t pk) {
  uint32_t lo = pk & 0xffffu, hi = pk >> 16;
  return lo > hi ? lo : hi;
}

// ---------------------------------------------------------------- E4M3
// Value of a scale byte 0x00..0x7E: normal (1+m/8)*2^(e-7), subnormal m*2^-9.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  uint32_t e = b >> 3, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}
// Nearest E4M3 byte of v >= 0 (ties to even), saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(v, 448.0f), 0.0f, 0, false) & 0xffu;
}

// ---------------------------------------------------------------- E2M1 pairs
// Packs E2M1(a), E2M1(b) (RNE, saturating, signed) into byte `sel` of `old`:
// a in the low nibble.
template <int sel>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, sel);
}

// ---------------------------------------------------------------- tables
// Per-tensor encode table, one entry per block-scale byte (0..126).
//
// Element code = E2M1(RN32(x / d)) with d = RN32(s*g).  The fast path uses
// y' = RN32(x * r), r = RN32(1/d), which differs from RN32(x/d) by < 2^-22.9
// relative.  E2M1 rounding of y only depends on where y lies against the
// seven grid midpoints b (0.25 ... 5), so y' gives the same code unless
// |x/d - b| <= 2^-22 b for some b.  Because x is bf16 (8 significant bits),
// for a given d at most one bf16 magnitude lies in each such window: the
// bf16 nearest to P = d*b (computed exactly in fp64).  build_entry records up
// to two such "danger" magnitudes; blocks that contain one are re-encoded by
// exact division.  Entries whose d is outside [2^-125, 2^125] (so 1/d could
// lose precision) are marked fully slow (r < 0).  d == 0 or +inf gives r = 0:
// x * 0 is a signed zero, which is exactly the recipe's code there.
struct Entry {
  float r;          // reciprocal of d (0: zero codes; < 0: exact division for the whole block)
  uint32_t danger;  // two bf16 magnitude patterns (low, high half); 0xFFFF = none
};

__device__ inline Entry build_entry(uint32_t sbyte, float g) {
  Entry e;
  e.danger = 0xffffffffu;
  const float s = e4m3_value(sbyte);
  const float d = s * g;
  if (d == 0.0f || __builtin_isinf(d)) { e.r = 0.0f; return e; }
  if (!(d >= 0x1p-125f && d <= 0x1p125f)) { e.r = -1.0f; return e; }
  e.r = 1.0f / d;   // correctly rounded (default HIP division)
  const float bnd[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  int nd = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) {
    const double P = (double)d * (double)bnd[k];       // exact (<= 27 significant bits)
    const uint64_t u = (uint64_t)__double_as_longlong(P);
    const int E = (int)((u >> 52) & 0x7ff) - 1023;
    if (E < -126) { e.r = -1.0f; return e; }
    const uint64_t low = u & ((1ull << 45) - 1);       // bits below the bf16 mantissa
    const uint64_t dist = low < (1ull << 44) ? low : (1ull << 45) - low;
    if (dist <= (1ull << 31)) {                        // a bf16 lies within 2^-22 of P
      const uint64_t ur = u + (1ull << 44);            // nearest bf16 grid point
      const int Er = (int)((ur >> 52) & 0x7ff) - 1023;
      if (Er > 127) continue;                          // beyond the largest finite bf16
      const uint32_t A = ((uint32_t)(Er + 127) << 7) | (uint32_t)((ur >> 45) & 0x7f);
      if (nd == 2) { e.r = -1.0f; return e; }
      e.danger = nd == 0 ? ((e.danger & 0xffff0000u) | A) : ((e.danger & 0xffffu) | (A << 16));
      ++nd;
    }
  }
  return e;
}

// Block-scale byte of a block from its amax (bf16 magnitude bits).
// Exact recipe: s = E4M3_RNE_SAT(RN32(bamax / d6)).  Fast path: RN32(bamax*r6)
// is within 2^-22.9 of the true quotient, so it rounds to the same E4M3 value
// unless it lies within 16 ulps of an E4M3 midpoint (mantissa pattern
// 1000...0 below the 3 kept bits) or in the subnormal E4M3 range; those take
// the exact division.  `exact_all` forces division (d6 outside [2^-125,2^125]).
__device__ __forceinline__ uint32_t block_scale_byte(uint32_t bam_bits, float d6, float r6, bool exact_all,
                                                     bool zero_all) {
  if (zero_all) return 0u;
  const float bam = __uint_as_float(bam_bits << 16);
  float qv = bam * r6;
  const uint32_t qb = __float_as_uint(qv);
  const int mid = (int)(qb & 0xfffffu) - 0x80000;
  const bool near = (mid >= -16 && mid <= 16) || (qv > 0.0f && qv < 0x1p-6f);
  if (exact_all || near) qv = bam / d6;
  return e4m3_rne_sat(qv);
}

// Encodes one 16-value block held as 8 words (element 2i in the low half of
// w[i]) given its table entry; returns the 8 code bytes as two words.
__device__ __forceinline__ void encode_block(const uint32_t (&w)[8], const Entry& en, uint32_t sbyte, float g,
                                             uint32_t& c0, uint32_t& c1) {
  const float r = en.r;
  if (r >= 0.0f) {
    c0 = fp4_pair<0>(0u, bf16_lo(w[0]) * r, bf16_hi(w[0]) * r);
    c0 = fp4_pair<1>(c0, bf16_lo(w[1]) * r, bf16_hi(w[1]) * r);
    c0 = fp4_pair<2>(c0, bf16_lo(w[2]) * r, bf16_hi(w[2]) * r);
    c0 = fp4_pair<3>(c0, bf16_lo(w[3]) * r, bf16_hi(w[3]) * r);
    c1 = fp4_pair<0>(0u, bf16_lo(w[4]) * r, bf16_hi(w[4]) * r);
    c1 = fp4_pair<1>(c1, bf16_lo(w[5]) * r, bf16_hi(w[5]) * r);
    c1 = fp4_pair<2>(c1, bf16_lo(w[6]) * r, bf16_hi(w[6]) * r);
    c1 = fp4_pair<3>(c1, bf16_lo(w[7]) * r, bf16_hi(w[7]) * r);
  }
  if (r < 0.0f || en.danger != 0xffffffffu) {
    // exact path: y = RN32(x / d) for every element (fully slow), or only for
    // the recorded danger magnitudes.
    const float d = e4m3_value(sbyte) * g;
    const bool all = r < 0.0f;
    const uint32_t A0 = en.danger & 0xffffu, A1 = en.danger >> 16;
    uint32_t out[2] = {c0, c1};
    if (all) { out[0] = 0u; out[1] = 0u; }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t xb = h ? (w[i] >> 16) : (w[i] & 0xffffu);
        const uint32_t ab = xb & 0x7fffu;
        if (all || ab == A0 || ab == A1) {
          const float x = __uint_as_float(xb << 16);
          const uint32_t code = fp4_pair<0>(0u, x / d, 0.0f) & 0xfu;
          const int sh = 8 * (i & 3) + 4 * h;
          out[i >> 2] = (out[i >> 2] & ~(0xfu << sh)) | (code << sh);
        }
      }
    }
    c0 = out[0];
    c1 = out[1];
  }
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

}  // namespace nvfp4

// ---------------------------------------------------------------- host side
namespace nvfp4host {
void set_hip_error(hipError_t e);
nvfp4_status check_device();                      // ENOTSUP unless the current device is gfx950
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int num_cus();                                    // compute units of the current device
}  // namespace nvfp4host

#define NVFP4_LAUNCH_CHECK()                       \
  do {                                             \
    hipError_t e_ = hipGetLastError();             \
    if (e_ != hipSuccess) {                        \
      nvfp4host::set_hip_error(e_);                \
      return NVFP4_EHIP;                           \
    }                                              \
  } while (0)
