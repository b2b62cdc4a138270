// Shared device helpers and host plumbing for libnvfp4 (gfx950 only).
//
// The E2M1 / E4M3 grids and the two-level scaling recipe are those of
// axbrief.com, "NVFP4: how NVIDIA pre-trained a 12B model on 10 trillion
// tokens", section "E2M1 format and two-level scaling".  The device code
// reaches the recipe's bits through gfx950's own conversion instructions
// (v_cvt_scalef32_pk_fp4_f32 rounds f32 to E2M1 to nearest-even with
// saturation, keeping the sign of zeros and underflows; v_cvt_pk_fp8_f32
// rounds to OCP E4M3 to nearest-even for inputs up to 464, so inputs are
// clamped to 448 first) and through fp64 reciprocals of the per-block
// divisors (see "exact quotients" below).
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

constexpr int kBlock = 16;             // values per E4M3 block scale
constexpr int kThreads = 256;          // threads per workgroup of the streaming kernels
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
// Nearest E4M3 byte of v >= 0 (ties to even), saturating at 448.  The
// conversion writes the byte of v and that of 0.0 (0x00) into the low half
// of a zero word, so the result is the byte itself.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(v, 448.0f), 0.0f, 0, false);
}

// ---------------------------------------------------------------- E2M1 pairs
// Packs E2M1(a), E2M1(b) (RNE, saturating, signed) into byte `sel` of `old`:
// a in the low nibble.
template <int sel>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, sel);
}

// ---------------------------------------------------------------- exact quotients
// Every quotient of the recipe has the form RN32(a / d) with a a bf16 value
// (8 significant bits) and d an fp32 value (24 significant bits): the block
// scale quotient bamax / d6 and the element quotient |x| / d.  Such a
// quotient is either exactly representable in fp32 or lies at least 2^-49
// (relative) away from every fp32 rounding midpoint: writing a = A 2^i,
// d = D 2^j with A, D odd, a/d is dyadic only when D divides A (and then has
// at most 8 significant bits); otherwise, for a midpoint m 2^(e-24) of the
// binade [2^e, 2^(e+1)), (a/d - m 2^(e-24)) D 2^j is a nonzero multiple of
// 2^min(i, e-24+j), which bounds the gap below by 2^-49 (a/d) either way.
// So y64 = RN64(a * RN64(1/d)), whose relative error is below 2^-52, rounds
// once to exactly RN32(a / d) -- E2M1 / E4M3 ties included -- with no
// division per element and no exception path.  fp64 multiplies and
// conversions run at the full VALU rate on gfx950.
//
// Per-tensor table: one fp64 reciprocal per block-scale byte (0..126).
// d == 0 (or +inf, from a huge caller scale) stores 0: x * 0 is the signed
// zero that the recipe prescribes there (x / inf = 0 too).
__device__ inline double recip_entry(uint32_t sbyte, float g) {
  const float d = e4m3_value(sbyte) * g;            // RN32(s * g)
  if (d == 0.0f || __builtin_isinf(d)) return 0.0;
  return 1.0 / (double)d;                           // RN64, correctly rounded
}

// RN32 of an fp64 value (one rounding; fp32 denormals are kept).
__device__ __forceinline__ float rn32(double v) { return (float)v; }

// Reciprocal of d6 = RN32(6 g) for the block-scale quotients; 0 when d6 is 0
// (all scales zero) or +inf (bamax / inf = 0).
__device__ __forceinline__ double recip_d6(float g) {
  const float d6 = 6.0f * g;
  if (d6 == 0.0f || __builtin_isinf(d6)) return 0.0;
  return 1.0 / (double)d6;
}

// Block-scale byte from the block amax (bf16 magnitude bits):
// s = E4M3_RNE_SAT(RN32(bamax / d6)).
__device__ __forceinline__ uint32_t block_scale_byte(uint32_t bam_bits, double r6) {
  const float bam = __uint_as_float(bam_bits << 16);
  return e4m3_rne_sat(rn32((double)bam * r6));
}

// RN32(x / d) for the two bf16 halves of a word, sign kept.
__device__ __forceinline__ float q_lo(uint32_t w, double r) { return rn32((double)bf16_lo(w) * r); }
__device__ __forceinline__ float q_hi(uint32_t w, double r) { return rn32((double)bf16_hi(w) * r); }

// ---------------------------------------------------------------- half blocks
// Streaming kernels give each lane HALF a block (8 values = 16 bytes of bf16),
// so consecutive lanes touch consecutive 16-byte chunks and every load and
// store instruction of a wave covers one contiguous run.  Lanes 2j and 2j+1
// hold the two halves of one block; they swap partial maxima with a DPP
// quad permutation.
__device__ __forceinline__ uint32_t half_absmax_bits(const u32x4 v) {
  uint32_t m = pk_absmax(pk_absmax(pk_absmax(pk_absmax(0u, v.x), v.y), v.z), v.w);
  return halves_max(m);
}
__device__ __forceinline__ uint32_t pair_max(uint32_t m) {
  // quad_perm(1,0,3,2): lane i reads lane i^1
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);
  return m > o ? m : o;
}

// Encodes 8 values (one half block) into 4 code bytes (element 2i in the low
// nibble of byte i) given the block's reciprocal r = RN64(1/d).
__device__ __forceinline__ uint32_t encode_half(const u32x4 w, double r) {
  // the four conversions write all four bytes, so the first one's other
  // bytes may start as anything (here the input word itself)
  uint32_t c = fp4_pair<0>(w.x, q_lo(w.x, r), q_hi(w.x, r));
  c = fp4_pair<1>(c, q_lo(w.y, r), q_hi(w.y, r));
  c = fp4_pair<2>(c, q_lo(w.z, r), q_hi(w.z, r));
  return fp4_pair<3>(c, q_lo(w.w, r), q_hi(w.w, r));
}

// Dequantizes 4 code bytes (8 values) with scale s and tensor scale g into 8
// bf16: RN32((E2M1 * s) * g) -> bf16 RNE.  The hardware decode yields the
// exact signed E2M1 value; E2M1 * s is exact in fp32.
__device__ __forceinline__ uint32_t deq_pair_bits(f32x2 f, float s, float g) {
  const __bf16 ha = (__bf16)((f.x * s) * g), hb = (__bf16)((f.y * s) * g);
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ u32x4 dequant_half(uint32_t codes, float s, float g) {
  u32x4 o;
  o.x = deq_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0), s, g);
  o.y = deq_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1), s, g);
  o.z = deq_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2), s, g);
  o.w = deq_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3), s, g);
  return o;
}

// gfx9 buffer resource word 3 (32-bit data format) for raw buffer loads and
// stores; accesses past the resource's extent read zero and write nothing.
constexpr int kBufferWord3 = 0x00020000;

// Cache-policy operand of a buffer load or store that streams data touched
// once: the non-temporal bit (bit 1 on gfx950), so the lines do not displace
// reused data in L2 and the last-level cache.  Measured on the fused
// quantize's buffer-to-LDS loads: 0.573 -> 0.530 ms over 1.88 GB of bf16.
constexpr int kStreamLoad = 2;

// Cache-policy operand of a load that must observe other compute units'
// atomic stores: sc1, the policy the compiler gives a relaxed agent-scope
// atomic load on gfx950 (the L2 of each XCD is not coherent with the others).
constexpr int kCoherentLoad = 16;

// ---------------------------------------------------------------- reductions
// Maximum over the 64 lanes of a wave (every lane active), returned
// wave-uniform.  DPP moves reduce each row of 16 lanes (quad swaps, then
// the half-row and row mirrors); four lane reads combine the rows.  No
// address registers are needed, unlike a shuffle through LDS permutes.
__device__ __forceinline__ uint32_t dpp_max(uint32_t v, int ctrl) {
  uint32_t o = 0;
  switch (ctrl) {   // the control word must be a compile-time constant
    case 0xB1: o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false); break;
    case 0x4E: o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false); break;
    case 0x141: o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false); break;
    default: o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false); break;
  }
  return v > o ? v : o;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max(v, 0xB1);    // quad_perm(1,0,3,2)
  v = dpp_max(v, 0x4E);    // quad_perm(2,3,0,1)
  v = dpp_max(v, 0x141);   // row_half_mirror
  v = dpp_max(v, 0x140);   // row_mirror: every lane holds its row's maximum
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// XCD-aware tile order.  The dispatcher hands workgroup i (linear id) to
// XCD i % 8, in order of i; each XCD has its own L2.  Giving XCD x a
// contiguous run of the T tiles (row-major over (m, n) tiles) makes the
// workgroups that share an A panel run on one XCD, so that panel is fetched
// into one L2 instead of eight.  Returns the tile index for workgroup lin.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_tile(int64_t lin, int64_t T) {
  const int64_t x = lin % kXcds, slot = lin / kXcds, per = T / kXcds, extra = T % kXcds;
  return x * per + (x < extra ? x : extra) + slot;
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
