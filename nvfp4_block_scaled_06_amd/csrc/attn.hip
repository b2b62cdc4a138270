// Decode-step attention over the NVFP4 KV cache: QK, softmax and P.V in one
// pass over the cache, split over workgroups along the tokens (flash-decoding
// style), then a small combine kernel.
//
// Decoding re-reads the whole KV cache every step, so storing it at 0.5625
// bytes per value cuts the bytes each step moves (theddari.com, "What is FP4
// quantization? KV cache in 4 bits", sections "KV cache size example" and
// "how does 4-bit KV change inference cost").  Here the cache is consumed in
// NVFP4 directly: K and V are decoded exactly in registers (E2M1 values from
// the hardware conversion, block and tensor scales applied in fp32), with
// nothing materialized in memory.
//
//   s_t  = scale * sum_d q[d] * Khat[t][d]
//   out  = sum_t exp(s_t - max s) Vhat[t] / sum_t exp(s_t - max s)
//
// Split kernel, grid (splits, kv_heads, layers): a workgroup takes the GRP
// query heads of one KV head (GQA) over one token range.  A token's head_dim
// values are split over LPT = head_dim/16 lanes, 16 values (one block) per
// lane: 8 code bytes and one scale byte of K and of V.  Each lane group keeps
// its own running softmax state (max, sum, 16 output values per head) over
// its tokens; the groups of a wave merge with lane shuffles and the waves of
// the workgroup through LDS, and the workgroup writes one partial (max, sum,
// head_dim unnormalized outputs) per query head.  The combine kernel merges
// the splits: out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "common.hpp"

namespace nvfp4 {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;

// Partial of one (layer, query head, split): max, sum, then head_dim outputs.
__host__ __device__ constexpr int64_t attn_partial_floats(int head_dim) { return 2 + head_dim; }

template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Sum over the LPT consecutive lanes of a token (LPT a power of two up to
// 16), all in DPP: lane i ^ 1, lane i ^ 2 (quad permutations), then the
// mirror within 8 lanes and within 16 lanes, each of which pairs the two
// halves of the group summed so far.
template <int LPT>
__device__ __forceinline__ float attn_group_sum(float v) {
  if (LPT >= 2) v += dpp_f<0xB1>(v);                   // quad_perm [1,0,3,2]
  if (LPT >= 4) v += dpp_f<0x4E>(v);                   // quad_perm [2,3,0,1]
  if (LPT >= 8) v += dpp_f<0x141>(v);                  // row_half_mirror
  if (LPT >= 16) v += dpp_f<0x140>(v);                 // row_mirror
  return v;
}

typedef __bf16 abf16x2 __attribute__((ext_vector_type(2)));

// Weights of two softmax states with maxima m and m2 after merging:
// a = exp(m - M), b = exp(m2 - M), M = max(m, m2) (exp(-inf) = 0 covers
// empty states).
__device__ __forceinline__ void attn_weights(float m, float m2, float& mn, float& a, float& b) {
  mn = fmaxf(m, m2);
  a = mn == -INFINITY ? 0.0f : __expf(m - mn);
  b = mn == -INFINITY ? 0.0f : __expf(m2 - mn);
}

template <int LPT, int GRP>
__global__ void __launch_bounds__(kAttnThreads) kv_attn_split_kernel(nvfp4_kv_cache c, const uint32_t* __restrict__ q,
                                                                     int q_heads, int64_t n, int64_t per_split,
                                                                     float scale, float* __restrict__ part) {
  constexpr int TPW = 64 / LPT;                          // tokens per wave
  constexpr int D = 16 * LPT;
  const int split = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int H = c.kv_heads;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int j = lane % LPT;                              // this lane's block of the token
  const int tg = lane / LPT;                             // token group within the wave
  // query slices: 16 values (8 bf16 pairs) of block j for each of the GRP heads
  uint32_t qv[GRP][8];
#pragma unroll
  for (int g = 0; g < GRP; ++g) {
    const u32x4* qp = (const u32x4*)(q + ((int64_t)l * q_heads + h * GRP + g) * (D / 2) + j * 8);
    const u32x4 a = qp[0], b = qp[1];
    qv[g][0] = a.x; qv[g][1] = a.y; qv[g][2] = a.z; qv[g][3] = a.w;
    qv[g][4] = b.x; qv[g][5] = b.y; qv[g][6] = b.z; qv[g][7] = b.w;
  }
  const float ks = c.k_g[l * H + h] * scale;            // tensor scale of K times the softmax scale
  const float gv = c.v_g[l * H + h];
  const int64_t row0 = ((int64_t)l * H + h) * c.capacity;
  const int64_t t0 = (int64_t)split * per_split;
  const int64_t t1 = std::min<int64_t>(n, t0 + per_split);
  // buffer resources over this split's tokens of (layer, head): codes 8 bytes
  // and one scale byte per lane and token; past t1 the loads read zeros
  const int64_t cnt = t1 > t0 ? t1 - t0 : 0;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.k + (row0 + t0) * (D / 2)), 0, (int)(cnt * (D / 2)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.v + (row0 + t0) * (D / 2)), 0, (int)(cnt * (D / 2)), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.k_sf + (row0 + t0) * LPT), 0, (int)(cnt * LPT), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rvs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.v_sf + (row0 + t0) * LPT), 0, (int)(cnt * LPT), kBufferWord3);

  float m[GRP], ls[GRP], o[GRP][16];
#pragma unroll
  for (int g = 0; g < GRP; ++g) {
    m[g] = -INFINITY;
    ls[g] = 0.0f;
#pragma unroll
    for (int d = 0; d < 16; ++d) o[g][d] = 0.0f;
  }
  // token u (relative to t0) of this lane group in trip i: (i * waves + wave) * TPW + tg
  const int64_t step = (int64_t)kAttnWaves * TPW;
  int64_t u = (int64_t)wave * TPW + tg;
  auto load = [&](int64_t uu, u32x2& kc, uint32_t& kb, u32x2& vc, uint32_t& vb) {
    const uint32_t e = uu < cnt ? (uint32_t)(uu * LPT + j) : 0x10000000u;     // past the extents: zeros
    kc = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, (int)(e * 8u), 0, 0));
    vc = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, (int)(e * 8u), 0, 0));
    kb = __builtin_amdgcn_raw_buffer_load_b8(rks, (int)e, 0, 0);
    vb = __builtin_amdgcn_raw_buffer_load_b8(rvs, (int)e, 0, 0);
  };
  u32x2 kc, vc;
  uint32_t kb, vb;
  load(u, kc, kb, vc, vb);
  // every lane of a wave runs the same trip count (the token group's own
  // tokens end at cnt; the trailing lanes compute on zeros and are masked)
  const int64_t trips = (cnt + step - 1) / step;
  for (int64_t it = 0; it < trips; ++it, u += step) {
    u32x2 kcn, vcn;
    uint32_t kbn, vbn;
    load(u + step, kcn, kbn, vcn, vbn);
    const bool live = u < cnt;
    // K block j: 16 exact E2M1 values as bf16 pairs, one scale
    const float sk = __builtin_amdgcn_cvt_f32_fp8((int)kb, 0);
    abf16x2 kp[8];
    kp[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(kc.x, 1.0f, 0);
    kp[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(kc.x, 1.0f, 1);
    kp[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(kc.x, 1.0f, 2);
    kp[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(kc.x, 1.0f, 3);
    kp[4] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(kc.y, 1.0f, 0);
    kp[5] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(kc.y, 1.0f, 1);
    kp[6] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(kc.y, 1.0f, 2);
    kp[7] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(kc.y, 1.0f, 3);
    float s[GRP];
#pragma unroll
    for (int g = 0; g < GRP; ++g) {
      float p = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) p = __builtin_amdgcn_fdot2_f32_bf16(kp[i], __builtin_bit_cast(abf16x2, qv[g][i]), p, false);
      s[g] = attn_group_sum<LPT>(p * sk) * ks;          // this token's logit, in every lane of the group
    }
    // V block j: 16 exact E2M1 values in f32
    const float sv = __builtin_amdgcn_cvt_f32_fp8((int)vb, 0) * gv;
    float v[16];
    f32x2 w;
    w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vc.x, 1.0f, 0); v[0] = w.x; v[1] = w.y;
    w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vc.x, 1.0f, 1); v[2] = w.x; v[3] = w.y;
    w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vc.x, 1.0f, 2); v[4] = w.x; v[5] = w.y;
    w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vc.x, 1.0f, 3); v[6] = w.x; v[7] = w.y;
    w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vc.y, 1.0f, 0); v[8] = w.x; v[9] = w.y;
    w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vc.y, 1.0f, 1); v[10] = w.x; v[11] = w.y;
    w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vc.y, 1.0f, 2); v[12] = w.x; v[13] = w.y;
    w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vc.y, 1.0f, 3); v[14] = w.x; v[15] = w.y;
#pragma unroll
    for (int g = 0; g < GRP; ++g) {
      const float sg = live ? s[g] : -INFINITY;         // lanes past the split add nothing
      // a new running max somewhere in the wave: rescale (a wave-uniform
      // branch, rare after the first tokens)
      if (__builtin_amdgcn_ballot_w64(sg > m[g])) {
        const float mn = fmaxf(m[g], sg);
        const float r = mn == -INFINITY ? 1.0f : __expf(m[g] - mn);
        ls[g] *= r;
#pragma unroll
        for (int d = 0; d < 16; ++d) o[g][d] *= r;
        m[g] = mn;
      }
      const float p = sg == -INFINITY ? 0.0f : __expf(sg - m[g]);
      ls[g] += p;
      const float pv = p * sv;
#pragma unroll
      for (int d = 0; d < 16; ++d) o[g][d] = __builtin_fmaf(pv, v[d], o[g][d]);
    }
    kc = kcn; kb = kbn; vc = vcn; vb = vbn;
  }
  // merge the token groups of the wave (lanes tg*LPT + j, same j), one
  // head and one output at a time
#pragma unroll
  for (int sh = LPT; sh < 64; sh <<= 1) {
#pragma unroll
    for (int g = 0; g < GRP; ++g) {
      float mn, a, b;
      attn_weights(m[g], __shfl_xor(m[g], sh, 64), mn, a, b);
      ls[g] = ls[g] * a + __shfl_xor(ls[g], sh, 64) * b;
#pragma unroll
      for (int d = 0; d < 16; ++d) o[g][d] = o[g][d] * a + __shfl_xor(o[g][d], sh, 64) * b;
      m[g] = mn;
    }
  }
  // merge the waves through LDS: lanes 0..LPT-1 of each wave hold its
  // state; then every thread merges (head, output) pairs of the workgroup,
  // with the loop state dead by then
  __shared__ float st[kAttnWaves][GRP][2 + D];
  if (lane < LPT) {
#pragma unroll
    for (int g = 0; g < GRP; ++g) {
      if (j == 0) {
        st[wave][g][0] = m[g];
        st[wave][g][1] = ls[g];
      }
#pragma unroll
      for (int d = 0; d < 16; ++d) st[wave][g][2 + 16 * j + d] = o[g][d];
    }
  }
  __syncthreads();
  const int splits = gridDim.x;
  for (int e = threadIdx.x; e < GRP * D; e += kAttnThreads) {
    const int g = e / D, d = e % D;
    float mx = st[0][g][0];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) mx = fmaxf(mx, st[w][g][0]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float a = st[w][g][0] == -INFINITY ? 0.0f : __expf(st[w][g][0] - mx);
      den = __builtin_fmaf(a, st[w][g][1], den);
      num = __builtin_fmaf(a, st[w][g][2 + d], num);
    }
    float* pp = part + (((int64_t)l * q_heads + h * GRP + g) * splits + split) * attn_partial_floats(D);
    if (d == 0) {
      pp[0] = mx;
      pp[1] = den;
    }
    pp[2 + d] = num;
  }
}

// ------------------------------------------------------------ MFMA split kernel
// The same split computation with both contractions on the matrix cores
// (head_dim D in {64, 128, 256}, up to 16 query heads per KV head).  A wave
// takes 32-token chunks; per chunk:
//  - QK: two v_mfma_f32_16x16x32_f16 tiles of 16 tokens x 16 heads, K
//    decoded exactly to f16 (E2M1 * s: at most 6 significant bits, within
//    f16's normal range) as the A operand; q as the B operand, scaled per
//    head by a power of two and rounded to f16 (exact except for elements
//    below 2^-28 of the head's largest).  The K dimension order is free,
//    so lane quarter qd takes head_dim values [qd D/4, (qd+1) D/4): one
//    contiguous code load per token.  Lane l ends with the logits of head
//    l % 16 for tokens 4 (l / 16) + i of each tile.
//  - online softmax per head across those lanes (fp32, exp of s - max).
//  - PV: v_mfma_f32_16x16x32_f16 per 16-column tile of the output, A = P
//    (heads x 32 tokens), B = V (32 tokens x 16 columns).  Token slot s of
//    lane l is token 16 (s / 4) + 4 (l / 16) + s % 4, so P comes straight
//    from the lane's own logits; P is split into f16 hi + lo parts (two
//    MFMAs) so it keeps about 21 bits.  V is decoded exactly to f16 (E2M1 *
//    s), written token-major to LDS and read back per column.
// The V tensor scale is applied once to the accumulated output.
constexpr int kMChunk = 32;                              // tokens per wave step

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef _Float16 h16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

template <int D>
struct AttnMfmaSmem {
  union {
    _Float16 v[kAttnWaves][kMChunk][D + 8];              // decoded V chunk of each wave (16-byte row padding)
    float st[kAttnWaves][16][2 + D];                     // per-wave softmax states for the final merge
  };
};

// Raw bytes one lane loads per chunk.
template <int D>
struct AttnRaw {
  uint32_t kc[2][D / 32];                                // K codes of the lane's quarter, tiles 0 and 1
  uint32_t ks[2];                                        // the D / 64 K scale bytes of the lane's quarter
  uint32_t vc[D / 16];                                   // V codes of the lane's half token
  uint32_t vs[D / 128 > 0 ? D / 128 : 1];                // V scale bytes of the half token (D / 32 bytes)
};

template <int W>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* dst) {
  // W words (W = 1, 2, 4, 8) from byte offset off
  if (W == 1) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kStreamLoad);
  } else if (W == 2) {
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kStreamLoad));
    dst[0] = v.x;
    dst[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < W; i += 4) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 4 * i), 0, kStreamLoad));
      dst[i] = v.x;
      dst[i + 1] = v.y;
      dst[i + 2] = v.z;
      dst[i + 3] = v.w;
    }
  }
}

// Byte offsets past every extent (extents stay below 2^30) read zeros.
constexpr uint32_t kAttnOutside = 0x80000000u;

template <int D>
__device__ __forceinline__ void attn_load(const __amdgpu_buffer_rsrc_t (&r)[4], int c0, int cnt, int lane,
                                          AttnRaw<D>& raw) {
  const int qd = lane >> 4;
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const int u = c0 + 16 * T + (lane & 15);
    const bool in = u < cnt;
    load_words<D / 32>(r[0], in ? (uint32_t)u * (D / 2) + qd * (D / 8) : kAttnOutside, raw.kc[T]);
    // the quarter's values [qd D/4, (qd+1) D/4) span blocks qd D/64 .. (qd+1) D/64 - 1
    const int so = (int)(in ? (uint32_t)u * (D / 16) + qd * (D / 64) : kAttnOutside);
    if (D == 64)
      raw.ks[T] = __builtin_amdgcn_raw_buffer_load_b8(r[1], so, 0, kStreamLoad);
    else if (D == 128)
      raw.ks[T] = __builtin_amdgcn_raw_buffer_load_b16(r[1], so, 0, kStreamLoad);
    else
      raw.ks[T] = __builtin_amdgcn_raw_buffer_load_b32(r[1], so, 0, kStreamLoad);
  }
  const int u = c0 + (lane >> 1);
  const bool in = u < cnt;
  load_words<D / 16>(r[2], in ? (uint32_t)u * (D / 2) + (lane & 1) * (D / 4) : kAttnOutside, raw.vc);
  if (D == 64)
    raw.vs[0] = __builtin_amdgcn_raw_buffer_load_b16(r[3], (int)(in ? (uint32_t)u * (D / 16) + (lane & 1) * 2 : kAttnOutside),
                                                     0, kStreamLoad);
  else
    load_words<(D / 128 > 0 ? D / 128 : 1)>(r[3], in ? (uint32_t)u * (D / 16) + (lane & 1) * (D / 32) : kAttnOutside,
                                            raw.vs);
}

// E4M3 byte b of a little-endian array of W words, decoded exactly (the
// word is picked with selects, so the array stays in registers).
template <int W>
__device__ __forceinline__ float e4m3_byte(const uint32_t (&words)[W], int b) {
  uint32_t w = words[0];
#pragma unroll
  for (int i = 1; i < W; ++i) w = (b >> 2) == i ? words[i] : w;
  return __builtin_amdgcn_cvt_f32_fp8((int)(w >> (8 * (b & 3))), 0);
}

// 8 E2M1 codes times scale s, exactly, as f16: the conversion applies s's
// power of two, one packed multiply its mantissa factor (1 + m/8).
__device__ __forceinline__ h16x8 dec8_f16(uint32_t w, float s) {
  const float mfs = __uint_as_float((__float_as_uint(s) & 0x007fffffu) | 0x3f800000u);
  const _Float16 mh = (_Float16)mfs;
  const h16x2 mf = {mh, mh};
  h16x8 o;
  h16x2 p;
  p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 0) * mf; o[0] = p.x; o[1] = p.y;
  p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 1) * mf; o[2] = p.x; o[3] = p.y;
  p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 2) * mf; o[4] = p.x; o[5] = p.y;
  p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, 3) * mf; o[6] = p.x; o[7] = p.y;
  return o;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__global__ void __launch_bounds__(kAttnThreads) kv_attn_mfma_kernel(nvfp4_kv_cache c, const uint32_t* __restrict__ q,
                                                                    int q_heads, int64_t n, int64_t per_split,
                                                                    float scale, float* __restrict__ part) {
  constexpr int KK = D / 32;                             // MFMA k steps of QK (8 values per lane each)
  constexpr int DT = D / 16;                             // output column tiles of PV
  const int split = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int H = c.kv_heads, GRP = q_heads / H;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int qd = lane >> 4, hl = lane & 15;              // lane quarter; head (QK B / P A row) or column
  __shared__ __attribute__((aligned(16))) AttnMfmaSmem<D> sm;
  // q as the QK B operand: head hl, values [qd D/4 + 8 kk, +8) for step kk
  // q as the QK B operand in f16: head hl's values times 2^cq, where cq puts
  // the head's largest |q| in [2^14, 2^15); exact for every element above
  // 2^-28 of that largest one.  The logits take 2^-cq back.
  u32x4 qw[KK];
  uint32_t qmax = 0u;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    qw[kk] = u32x4{0u, 0u, 0u, 0u};
    if (hl < GRP) qw[kk] = *(const u32x4*)(q + ((int64_t)l * q_heads + h * GRP + hl) * (D / 2) + qd * (D / 8) + 4 * kk);
    qmax = halves_max(pk_absmax(pk_absmax(pk_absmax(pk_absmax(qmax, qw[kk].x), qw[kk].y), qw[kk].z), qw[kk].w));
  }
  qmax = max(qmax, (uint32_t)__shfl_xor((int)qmax, 16, 64));
  qmax = max(qmax, (uint32_t)__shfl_xor((int)qmax, 32, 64));
  const int qe = (int)(qmax >> 7);                       // biased exponent of the head's largest |q|
  const int cq = qe == 0 ? 0 : std::min(std::max(141 - qe, -100), 100);
  // the sign of the softmax scale goes into q (exact), so the logits in
  // MFMA units order like the scaled ones and the running max is taken on
  // them directly
  const float qs = __uint_as_float((uint32_t)(cq + 127) << 23 | (scale < 0.0f ? 0x80000000u : 0u));
  h16x8 qb[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const uint32_t w[4] = {qw[kk].x, qw[kk].y, qw[kk].z, qw[kk].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qb[kk][2 * i] = (_Float16)(bf16_lo(w[i]) * qs);
      qb[kk][2 * i + 1] = (_Float16)(bf16_hi(w[i]) * qs);
    }
  }
  // logit = ks * (MFMA sum); exp(logit - max) = exp2((sum - max sum) * kl)
  const float ks = c.k_g[l * H + h] * fabsf(scale) * __uint_as_float((uint32_t)(127 - cq) << 23);
  const float kl = fmaxf(ks * 1.44269504f, 1.17549435e-38f);   // > 0: masked tokens give -inf, not NaN
  const float gv = c.v_g[l * H + h];
  const int64_t row0 = ((int64_t)l * H + h) * c.capacity;
  const int64_t t0 = (int64_t)split * per_split;
  const int64_t t1 = std::min<int64_t>(n, t0 + per_split);
  const int64_t cnt = t1 > t0 ? t1 - t0 : 0;
  const __amdgpu_buffer_rsrc_t rs[4] = {
      __builtin_amdgcn_make_buffer_rsrc((void*)(c.k + (row0 + t0) * (D / 2)), 0, (int)(cnt * (D / 2)), kBufferWord3),
      __builtin_amdgcn_make_buffer_rsrc((void*)(c.k_sf + (row0 + t0) * (D / 16)), 0, (int)(cnt * (D / 16)), kBufferWord3),
      __builtin_amdgcn_make_buffer_rsrc((void*)(c.v + (row0 + t0) * (D / 2)), 0, (int)(cnt * (D / 2)), kBufferWord3),
      __builtin_amdgcn_make_buffer_rsrc((void*)(c.v_sf + (row0 + t0) * (D / 16)), 0, (int)(cnt * (D / 16)), kBufferWord3)};

  float m = -INFINITY, lsum = 0.0f;                      // head hl: running max, this lane's partial sum
  f32x4v o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
  _Float16(*vs)[D + 8] = sm.v[wave];
  AttnRaw<D> cur;
  // token counts and offsets within a split are 32-bit: the host keeps
  // n * head_dim / 2 below 2^30
  const int cnt32 = (int)cnt;
  int c0 = wave * kMChunk;
  attn_load<D>(rs, c0, cnt32, lane, cur);
  for (; c0 < cnt32; c0 += kAttnWaves * kMChunk) {
    AttnRaw<D> nxt;
    attn_load<D>(rs, c0 + kAttnWaves * kMChunk, cnt32, lane, nxt);
    // ---- QK: logits of head hl, tokens 16 T + 4 qd + i
    f32x4v sacc[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      sacc[T] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const float sk = __builtin_amdgcn_cvt_f32_fp8((int)(cur.ks[T] >> (8 * (kk / 2))), 0);   // block kk / 2 of the quarter
        sacc[T] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dec8_f16(cur.kc[T][kk], sk), qb[kk], sacc[T], 0, 0, 0);
      }
    }
    // ---- V chunk into LDS: lane (token lane / 2, half lane % 2)
    {
      const int tk = lane >> 1, hf = lane & 1;
#pragma unroll
      for (int w = 0; w < D / 16; ++w) {
        const float sv = e4m3_byte(cur.vs, w / 2);
        *(h16x8*)&vs[tk][hf * (D / 2) + 8 * w] = dec8_f16(cur.vc[w], sv);
      }
    }
    // ---- online softmax for head hl over this chunk, in MFMA units (the
    // running max m too); kl turns differences into base-2 exponents
    float sv8[8];
    float cmax = -INFINITY;
    const int rem = std::min(cnt32 - c0, kMChunk);                 // tokens of the chunk inside the split
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) sv8[s8] = sacc[s8 >> 2][s8 & 3];
    if (rem < kMChunk) {                                           // the split's last chunk
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8)
        if (16 * (s8 >> 2) + 4 * qd + (s8 & 3) >= rem) sv8[s8] = -INFINITY;
    }
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) cmax = fmaxf(cmax, sv8[s8]);
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float mn = fmaxf(m, cmax);
    const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((m - mn) * kl);
    m = mn;
    float p8[8];
    const float mref = mn == -INFINITY ? 0.0f : mn;               // exp(-inf - mref) = 0 for masked tokens
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) p8[s8] = __builtin_amdgcn_exp2f((sv8[s8] - mref) * kl);
    float psum = p8[0];
#pragma unroll
    for (int s8 = 1; s8 < 8; ++s8) psum += p8[s8];
    lsum = lsum * alpha + psum;
    if (__builtin_amdgcn_ballot_w64(hl < GRP && alpha != 1.0f)) {   // rescale the output rows (heads 4 qd + i)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = __shfl(alpha, 4 * qd + i, 64);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt][i] *= a;
      }
    }
    // ---- P (head hl x token slots 8 qd .. 8 qd + 7) in f16 hi + lo: hi is
    // p with its low 13 mantissa bits cleared (exact in f16 for p >= 2^-14),
    // lo = p - hi is exact in fp32 and rounds to f16 with error at most 2^-22 p.
    // Rows of heads hl >= GRP (zero queries) hold finite values and feed only
    // output rows that are never stored.
    h16x8 ph, pl;
#pragma unroll
    for (int s8 = 0; s8 < 8; s8 += 2) {
      const float h0 = __uint_as_float(__float_as_uint(p8[s8]) & 0xFFFFE000u);
      const float h1 = __uint_as_float(__float_as_uint(p8[s8 + 1]) & 0xFFFFE000u);
      ph[s8] = (_Float16)h0;
      ph[s8 + 1] = (_Float16)h1;
      pl[s8] = (_Float16)(p8[s8] - h0);
      pl[s8 + 1] = (_Float16)(p8[s8 + 1] - h1);
    }
    wave_lds_sync();                                     // V chunk written
    // ---- PV: column tile dt, B[slot][column hl] = V[token(slot)][16 dt + hl].
    // ds_read_b64_tr_b16 hands lane j of a 16-lane group element b of the
    // 8-byte piece that lane 4 i + j / 4 addressed, as its element i: lane
    // k of quarter qd addresses V[token 16 r + 4 qd + k / 4][16 dt + 4 (k % 4)]
    // for slots 4 r .. 4 r + 3 (r = 0, 1).
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const h16x4 b0 = __builtin_bit_cast(h16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)&vs[4 * qd + (hl >> 2)][16 * dt + 4 * (hl & 3)]));
      const h16x4 b1 = __builtin_bit_cast(h16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)&vs[16 + 4 * qd + (hl >> 2)][16 * dt + 4 * (hl & 3)]));
      const h16x8 vb = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph, vb, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, vb, o[dt], 0, 0, 0);
    }
    wave_lds_sync();                                     // reads done before the next chunk's writes
    cur = nxt;
  }
  // ---- this wave's state: head hl's sum over the four quarters
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  __syncthreads();                                       // every wave is done with its V buffer (st aliases it)
  if (lane < GRP) {
    sm.st[wave][lane][0] = m == -INFINITY ? m : m * ks;   // the max logit, for the merges
    sm.st[wave][lane][1] = lsum;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hd = 4 * qd + i;                           // output row of o[.][i]
    if (hd < GRP) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) sm.st[wave][hd][2 + 16 * dt + hl] = o[dt][i] * gv;
    }
  }
  __syncthreads();
  const int splits = gridDim.x;
  for (int e = threadIdx.x; e < GRP * D; e += kAttnThreads) {
    const int g = e / D, d = e % D;
    float mx = sm.st[0][g][0];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) mx = fmaxf(mx, sm.st[w][g][0]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float a = sm.st[w][g][0] == -INFINITY ? 0.0f : __expf(sm.st[w][g][0] - mx);
      den = __builtin_fmaf(a, sm.st[w][g][1], den);
      num = __builtin_fmaf(a, sm.st[w][g][2 + d], num);
    }
    float* pp = part + (((int64_t)l * q_heads + h * GRP + g) * splits + split) * attn_partial_floats(D);
    if (d == 0) {
      pp[0] = mx;
      pp[1] = den;
    }
    pp[2 + d] = num;
  }
}

// grid (q_heads, layers), head_dim threads: merges the splits of one query head.
__global__ void kv_attn_combine_kernel(const float* __restrict__ part, int splits, int head_dim,
                                       float* __restrict__ out) {
  const int hq = blockIdx.x, l = blockIdx.y, d = threadIdx.x;
  const int q_heads = gridDim.x;
  const float* pp = part + ((int64_t)l * q_heads + hq) * splits * attn_partial_floats(head_dim);
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, pp[s * attn_partial_floats(head_dim)]);
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const float* ps = pp + s * attn_partial_floats(head_dim);
    const float w = ps[0] == -INFINITY ? 0.0f : __expf(ps[0] - M);
    den = __builtin_fmaf(w, ps[1], den);
    num = __builtin_fmaf(w, ps[2 + d], num);
  }
  out[((int64_t)l * q_heads + hq) * head_dim + d] = num / den;
}

}  // namespace nvfp4

namespace {

using namespace nvfp4;

constexpr int kAttnMaxBlocksPerCU = 2048 / kAttnThreads;   // 32 waves per CU

typedef void (*attn_kernel_t)(nvfp4_kv_cache, const uint32_t*, int, int64_t, int64_t, float, float*);

// Index of (head_dim/16, q_heads/kv_heads) in the instantiation table, or
// -1 when the shape has no kernel.
int attn_index(const nvfp4_kv_cache* c, int32_t q_heads) {
  const int lpt = c->head_dim / 16, grp = q_heads / c->kv_heads;
  const int li = lpt == 1 ? 0 : lpt == 2 ? 1 : lpt == 4 ? 2 : lpt == 8 ? 3 : lpt == 16 ? 4 : -1;
  const int gi = grp == 1 ? 0 : grp == 2 ? 1 : grp == 4 ? 2 : grp == 8 ? 3 : -1;
  return li < 0 || gi < 0 ? -1 : li * 4 + gi;
}

const attn_kernel_t kAttnKernels[20] = {
    kv_attn_split_kernel<1, 1>,  kv_attn_split_kernel<1, 2>,  kv_attn_split_kernel<1, 4>,  kv_attn_split_kernel<1, 8>,
    kv_attn_split_kernel<2, 1>,  kv_attn_split_kernel<2, 2>,  kv_attn_split_kernel<2, 4>,  kv_attn_split_kernel<2, 8>,
    kv_attn_split_kernel<4, 1>,  kv_attn_split_kernel<4, 2>,  kv_attn_split_kernel<4, 4>,  kv_attn_split_kernel<4, 8>,
    kv_attn_split_kernel<8, 1>,  kv_attn_split_kernel<8, 2>,  kv_attn_split_kernel<8, 4>,  kv_attn_split_kernel<8, 8>,
    kv_attn_split_kernel<16, 1>, kv_attn_split_kernel<16, 2>, kv_attn_split_kernel<16, 4>, kv_attn_split_kernel<16, 8>,
};

// Resident workgroups per CU of a split kernel (register and LDS limits),
// asked of the runtime once per instantiation.
int attn_blocks_per_cu(int idx) {
  static std::atomic<int> cache[20];
  int b = cache[idx].load(std::memory_order_relaxed);
  if (b > 0) return b;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, reinterpret_cast<const void*>(kAttnKernels[idx]),
                                                   kAttnThreads, 0) != hipSuccess || b <= 0)
    b = 1;
  b = std::min(b, kAttnMaxBlocksPerCU);
  cache[idx].store(b, std::memory_order_relaxed);
  return b;
}

// The same for the MFMA kernels (head_dim 64, 128, 256).
int attn_mfma_blocks_per_cu(int head_dim) {
  static std::atomic<int> cache[3];
  const int idx = head_dim == 64 ? 0 : head_dim == 128 ? 1 : 2;
  int b = cache[idx].load(std::memory_order_relaxed);
  if (b > 0) return b;
  const void* fn = idx == 0 ? reinterpret_cast<const void*>(kv_attn_mfma_kernel<64>)
                   : idx == 1 ? reinterpret_cast<const void*>(kv_attn_mfma_kernel<128>)
                              : reinterpret_cast<const void*>(kv_attn_mfma_kernel<256>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, fn, kAttnThreads, 0) != hipSuccess || b <= 0) b = 1;
  b = std::min(b, kAttnMaxBlocksPerCU);
  cache[idx].store(b, std::memory_order_relaxed);
  return b;
}

// Splits per (layer, KV head): one full round of resident workgroups over
// the chip (no partly filled second round), at least 64 tokens per split.
int attn_splits(const nvfp4_kv_cache* c, int64_t n, int blocks_per_cu) {
  const int64_t pairs = (int64_t)c->layers * c->kv_heads;
  const int64_t want = std::max<int64_t>(1, ((int64_t)nvfp4host::num_cus() * blocks_per_cu + pairs - 1) / pairs);
  const int64_t most = std::max<int64_t>(1, (n + 63) / 64);
  return (int)std::min<int64_t>(std::min(want, most), 1024);
}

size_t attn_workspace(const nvfp4_kv_cache* c, int32_t q_heads, int splits) {
  return (size_t)c->layers * (size_t)q_heads * (size_t)splits * (size_t)attn_partial_floats(c->head_dim) *
         sizeof(float);
}

}  // namespace

extern "C" {

size_t nvfp4_kv_attention_workspace_bytes(const nvfp4_kv_cache* c, int32_t q_heads, int64_t n) {
  if (!c || c->layers <= 0 || c->kv_heads <= 0 || c->head_dim <= 0 || q_heads <= 0 || n <= 0) return 0;
  // an upper bound over every occupancy the split kernels can have
  return attn_workspace(c, q_heads, attn_splits(c, n, kAttnMaxBlocksPerCU));
}

nvfp4_status nvfp4_kv_decode_attention(const nvfp4_kv_cache* c, const uint16_t* q, int32_t q_heads, int64_t n,
                                       float scale, float* out, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (!c) return NVFP4_EINVAL;
  if (c->layers <= 0 || c->kv_heads <= 0 || c->head_dim <= 0 || c->capacity < 0 || c->head_dim % kBlock)
    return NVFP4_EINVAL;
  if (c->kv_heads > 65535 || c->layers > 65535) return NVFP4_EINVAL;
  if (!c->k || !c->v || !c->k_sf || !c->v_sf || !c->k_g || !c->v_g) return NVFP4_EINVAL;
  if (q_heads <= 0 || q_heads % c->kv_heads) return NVFP4_EINVAL;
  if (n <= 0 || n > c->capacity) return NVFP4_EINVAL;             // softmax needs at least one token
  if (!q || !out || !std::isfinite(scale)) return NVFP4_EINVAL;
  const int grp = q_heads / c->kv_heads;
  const bool mfma = (c->head_dim == 64 || c->head_dim == 128 || c->head_dim == 256) && grp <= 16;
  const int idx = attn_index(c, q_heads);
  if (!mfma && idx < 0) return NVFP4_ENOTSUP;
  if (n * (c->head_dim / 2) >= (INT64_C(1) << 30)) return NVFP4_EINVAL;   // 32-bit buffer offsets
  if (!nvfp4host::aligned16(q) || !nvfp4host::aligned16(out) || !nvfp4host::aligned16(c->k) ||
      !nvfp4host::aligned16(c->v))
    return NVFP4_EALIGN;
  if ((reinterpret_cast<uintptr_t>(c->k_g) & 3u) || (reinterpret_cast<uintptr_t>(c->v_g) & 3u)) return NVFP4_EALIGN;
  if (!workspace || workspace_bytes < nvfp4_kv_attention_workspace_bytes(c, q_heads, n)) return NVFP4_EWORKSPACE;
  if (!nvfp4host::aligned16(workspace)) return NVFP4_EALIGN;
  nvfp4_status st = nvfp4host::check_device();
  if (st) return st;
  const int splits = attn_splits(c, n, mfma ? attn_mfma_blocks_per_cu(c->head_dim) : attn_blocks_per_cu(idx));
  const int64_t per_split = (n + splits - 1) / splits;
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid(splits, c->kv_heads, c->layers);
  const uint32_t* qa = (const uint32_t*)q;
  float* part = (float*)workspace;
  if (!mfma)
    kAttnKernels[idx]<<<grid, kAttnThreads, 0, s>>>(*c, qa, q_heads, n, per_split, scale, part);
  else if (c->head_dim == 64)
    kv_attn_mfma_kernel<64><<<grid, kAttnThreads, 0, s>>>(*c, qa, q_heads, n, per_split, scale, part);
  else if (c->head_dim == 128)
    kv_attn_mfma_kernel<128><<<grid, kAttnThreads, 0, s>>>(*c, qa, q_heads, n, per_split, scale, part);
  else
    kv_attn_mfma_kernel<256><<<grid, kAttnThreads, 0, s>>>(*c, qa, q_heads, n, per_split, scale, part);
  NVFP4_LAUNCH_CHECK();
  kv_attn_combine_kernel<<<dim3(q_heads, c->layers), c->head_dim, 0, s>>>(part, splits, c->head_dim, out);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

}  // extern "C"
