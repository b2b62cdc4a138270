// NVFP4 KV cache: append (encode new K/V tokens into the cache layout), read
// (dequantize a token range) and the decode-step QK sweep.
//
// The KV cache stores K and V in NVFP4 at 0.5625 bytes per value and decoding
// re-reads it every step, so a smaller cache means fewer bytes per step
// (theddari.com, "What is FP4 quantization? KV cache in 4 bits", sections "KV
// cache size example" and "how does 4-bit KV change inference cost").
//
// Cache layout: codes [layers][kv_heads][capacity][head_dim/2], block scales
// [layers][kv_heads][capacity][head_dim/16]; one (layer, head) owns a
// contiguous run of tokens, so appends write and decode sweeps read long
// contiguous stretches.  Each (layer, head) has its own fixed tensor scale
// (k_g / v_g), so one workgroup serves one (layer, head, K|V) and builds that
// scale's encode table once.
#include <algorithm>

#include "common.hpp"

namespace nvfp4 {

// grid (tiles, kv_heads, 2*layers): z = 2*layer + (0: K, 1: V).  Work unit:
// half block j of the chunk's rows for this (layer, head), j in [0, n*R),
// R = head_dim/8 half blocks per token row.  Lane j of a wave chunk maps to
// token j / R, half block j % R (shifts when kPow2).  Input rows of one head
// are head_dim*kv_heads apart; cache rows of consecutive tokens are
// contiguous, so the code stores of a wave form one run.  Each wave takes
// kKVU chunks of 64 half blocks per trip with all their loads in flight, and
// the workgroup's first loads are issued before it builds the scale's table.
constexpr int kKVU = 2;
constexpr int kKVReadU = 4;   // half blocks per lane per trip of kv_read (loads in flight)

template <bool kPow2>
__device__ __forceinline__ void kv_append_load(const u32x4* __restrict__ src, int64_t base, int64_t total,
                                               uint32_t R, int log2r, int64_t in_stride, u32x4 (&v)[kKVU]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kKVU; ++u) {
    const int64_t j = base + u * 64 + lane;
    uint32_t t, r;
    if (kPow2) {
      t = (uint32_t)(j >> log2r);
      r = (uint32_t)j & (R - 1);
    } else {
      t = (uint32_t)(j / R);
      r = (uint32_t)(j - (int64_t)t * R);
    }
    v[u] = j < total ? __builtin_nontemporal_load(src + ((int64_t)t * in_stride + r)) : u32x4{0u, 0u, 0u, 0u};
  }
}

template <bool kPow2>
__global__ void __launch_bounds__(kThreads) kv_append_kernel(nvfp4_kv_cache c, int64_t start, int64_t n, int log2r,
                                                             const u32x4* __restrict__ k_new,
                                                             const u32x4* __restrict__ v_new) {
  const int h = blockIdx.y;
  const int l = blockIdx.z >> 1;
  const bool is_v = blockIdx.z & 1;
  const int H = c.kv_heads;
  const uint32_t R = (uint32_t)c.head_dim / 8;
  const u32x4* src = (is_v ? v_new : k_new) + ((int64_t)l * n * H + h) * R;    // token 0 of (l, h)
  uint32_t* dq = (uint32_t*)(is_v ? c.v : c.k) + (((int64_t)l * H + h) * c.capacity + start) * R;
  uint8_t* dsf = (is_v ? c.v_sf : c.k_sf) + (((int64_t)l * H + h) * c.capacity + start) * (R / 2);
  const int64_t total = n * (int64_t)R;
  const int lane = threadIdx.x & 63;
  const int64_t in_stride = (int64_t)H * R;                                     // between tokens
  const int64_t span = 64 * kKVU;
  const int64_t stride = (int64_t)gridDim.x * (kThreads / 64) * span;
  int64_t base = ((int64_t)blockIdx.x * (kThreads / 64) + wave_id()) * span;
  u32x4 v[kKVU];
  kv_append_load<kPow2>(src, base, total, R, log2r, in_stride, v);
  const float g = (is_v ? c.v_g : c.k_g)[l * H + h];
  __shared__ double table[128];
  for (uint32_t j = threadIdx.x; j < 127u; j += kThreads) table[j] = recip_entry(j, g);
  __syncthreads();
  const double r6 = recip_d6(g);
  for (; base < total; base += stride) {
#pragma unroll
    for (int u = 0; u < kKVU; ++u) {
      const int64_t j = base + u * 64 + lane;
      const uint32_t sbyte = block_scale_byte(pair_max(half_absmax_bits(v[u])), r6);
      const uint32_t code = encode_half(v[u], table[sbyte]);
      if (j < total) {
        dq[j] = code;
        if ((lane & 1) == 0) dsf[j >> 1] = (uint8_t)sbyte;
      }
    }
    if (base + stride < total) kv_append_load<kPow2>(src, base + stride, total, R, log2r, in_stride, v);
  }
}

__device__ __forceinline__ uint32_t kv_dequant_pair(float2 f, float s, float g) {
  const __bf16 ha = (__bf16)((f.x * s) * g), hb = (__bf16)((f.y * s) * g);
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

__device__ __forceinline__ u32x4 kv_dequant_half(uint32_t codes, float s, float g) {
  u32x4 o;
  f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  o.x = kv_dequant_pair(make_float2(f0.x, f0.y), s, g);
  o.y = kv_dequant_pair(make_float2(f1.x, f1.y), s, g);
  o.z = kv_dequant_pair(make_float2(f2.x, f2.y), s, g);
  o.w = kv_dequant_pair(make_float2(f3.x, f3.y), s, g);
  return o;
}

// grid (tiles, kv_heads, 2*nlayers); out [nlayers][H][n][D] bf16, stored
// non-temporal (written once, not read back here).
__global__ void __launch_bounds__(kThreads) kv_read_kernel(nvfp4_kv_cache c, int layer0, int64_t t0, int64_t n,
                                                           u32x4* __restrict__ k_out, u32x4* __restrict__ v_out) {
  const int h = blockIdx.y;
  const int li = blockIdx.z >> 1;
  const bool is_v = blockIdx.z & 1;
  u32x4* out = is_v ? v_out : k_out;
  if (!out) return;
  const int l = layer0 + li;
  const int H = c.kv_heads, hpr = c.head_dim / 8;                  // half blocks per token
  const float g = (is_v ? c.v_g : c.k_g)[l * H + h];
  // tokens [t0, t0 + n) of (l, h) are contiguous in the cache and in the
  // output: one lane per half block (4 code bytes in, 16 bf16 bytes out), so
  // a wave's stores cover 1 KiB without gaps
  const int64_t row0 = ((int64_t)l * H + h) * c.capacity + t0;
  const uint32_t* sq = (const uint32_t*)(is_v ? c.v : c.k) + row0 * hpr;
  const uint8_t* ssf = (is_v ? c.v_sf : c.k_sf) + row0 * (hpr / 2);
  u32x4* o = out + ((int64_t)li * H + h) * n * hpr;
  const int64_t nh = n * hpr;
  const int64_t step = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kKVReadU - 1) * step < nh; i += kKVReadU * step) {
    uint32_t cw[kKVReadU];
    uint8_t sb[kKVReadU];
#pragma unroll
    for (int u = 0; u < kKVReadU; ++u) {
      cw[u] = __builtin_nontemporal_load(sq + i + u * step);
      sb[u] = ssf[(i + u * step) >> 1];
    }
#pragma unroll
    for (int u = 0; u < kKVReadU; ++u)
      __builtin_nontemporal_store(kv_dequant_half(cw[u], e4m3_value(sb[u]), g), o + i + u * step);
  }
  for (; i < nh; i += step) __builtin_nontemporal_store(kv_dequant_half(sq[i], e4m3_value(ssf[i >> 1]), g), o + i);
}

// Decode-step QK: grid (token tiles, kv_heads, layers).  The grp query heads
// of one KV head (GQA) are staged in LDS as f32; each lane takes one
// (token, block) pair, decodes its 16 K values exactly (E2M1 * s in f32) and
// accumulates grp partial dot products, which the bpr lanes of a token then
// sum with shuffles.  logit = g * sum (exact K products, fp32 accumulation).
constexpr int kQKMaxLds = 16 * 256;   // grp * head_dim floats

__global__ void __launch_bounds__(kThreads) kv_decode_qk_kernel(nvfp4_kv_cache c, const uint16_t* __restrict__ q,
                                                                int q_heads, int64_t n, float* __restrict__ logits) {
  const int h = blockIdx.y, l = blockIdx.z;
  const int H = c.kv_heads, D = c.head_dim, bpr = D / kBlock;
  const int grp = q_heads / H;
  __shared__ float qs[kQKMaxLds];
  for (int i = threadIdx.x; i < grp * D; i += kThreads) {
    const int hq = h * grp + i / D;
    qs[i] = __uint_as_float((uint32_t)q[((int64_t)l * q_heads + hq) * D + (i % D)] << 16);
  }
  __syncthreads();
  const float g = c.k_g[l * H + h];
  const u32x2* kq = (const u32x2*)c.k;
  const int64_t row0 = ((int64_t)l * H + h) * c.capacity;
  // bpr is a power of two dividing 64 (validated on the host), so every token's
  // lanes sit in one wave and the tile loop keeps whole tokens per iteration.
  const int64_t tokens_per_iter = kThreads / bpr;
  for (int64_t t0 = (int64_t)blockIdx.x * tokens_per_iter; t0 < n; t0 += (int64_t)gridDim.x * tokens_per_iter) {
    const int64_t t = t0 + threadIdx.x / bpr;
    const int j = threadIdx.x % bpr;
    float kv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) kv[e] = 0.0f;
    if (t < n) {
      const u32x2 cw = kq[(row0 + t) * bpr + j];
      const float s = e4m3_value(c.k_sf[(row0 + t) * bpr + j]);
      const f32x2 f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw.x, 1.0f, 0);
      const f32x2 f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw.x, 1.0f, 1);
      const f32x2 f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw.x, 1.0f, 2);
      const f32x2 f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw.x, 1.0f, 3);
      const f32x2 f4 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw.y, 1.0f, 0);
      const f32x2 f5 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw.y, 1.0f, 1);
      const f32x2 f6 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw.y, 1.0f, 2);
      const f32x2 f7 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw.y, 1.0f, 3);
      kv[0] = f0.x * s; kv[1] = f0.y * s; kv[2] = f1.x * s; kv[3] = f1.y * s;
      kv[4] = f2.x * s; kv[5] = f2.y * s; kv[6] = f3.x * s; kv[7] = f3.y * s;
      kv[8] = f4.x * s; kv[9] = f4.y * s; kv[10] = f5.x * s; kv[11] = f5.y * s;
      kv[12] = f6.x * s; kv[13] = f6.y * s; kv[14] = f7.x * s; kv[15] = f7.y * s;
    }
    for (int hq = 0; hq < grp; ++hq) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc = __builtin_fmaf(qs[hq * D + 16 * j + e], kv[e], acc);
      for (int off = 1; off < bpr; off <<= 1) acc += __shfl_xor(acc, off, 64);
      if (t < n && j == 0) logits[((int64_t)l * q_heads + h * grp + hq) * n + t] = acc * g;
    }
  }
}

// Decode-step QK, register-resident queries.  Each token's head_dim K
// values are split over LPT = head_dim/32 consecutive lanes (32 values = 16
// code bytes + 2 scale bytes per lane), so a wave reads 64/LPT tokens' codes
// as one contiguous run.  Every lane keeps its 32-value slice of the GRP
// query heads of this KV head (GQA) in registers as bf16 pairs.  K is decoded
// exactly to bf16 pairs (E2M1 values; v_cvt_scalef32_pk_bf16_fp4) and
// contracted with v_dot2_f32_bf16 (bf16 x bf16 products are exact in fp32);
// each 16-value block's partial is scaled by its s, the LPT lanes of a token
// are summed with DPP butterflies, and g is applied once per logit.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kQKGroups = 4;   // token groups per trip of kv_qk_kernel (loads in flight)

template <int sel>
__device__ __forceinline__ bf16x2 kpair(uint32_t codes) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, sel);
}

// First product of a dot chain, a.x*b.x + a.y*b.y + 0, in the three-operand
// form (the two-operand form the compiler picks needs a zeroed accumulator).
__device__ __forceinline__ float dot2_first(bf16x2 a, bf16x2 b) {
  float r;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// (old 0 with bound_ctrl lets the compiler fold each move into the add as a
// DPP operand: one instruction per butterfly step)
template <int LPT>
__device__ __forceinline__ float lane_group_sum(float v) {
  if (LPT >= 2)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  if (LPT >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  if (LPT >= 8) v += __shfl_xor(v, 4, 64);
  return v;
}

template <int LPT, int GRP>
__global__ void __launch_bounds__(kThreads) kv_qk_kernel(nvfp4_kv_cache c, const uint32_t* __restrict__ q,
                                                         int q_heads, int64_t n64, float* __restrict__ logits) {
  constexpr int TPW = 64 / LPT;                        // tokens per wave
  constexpr int U = kQKGroups;                         // token groups per trip
  const int h = blockIdx.y, l = blockIdx.z;
  const int H = c.kv_heads;
  const int lane = threadIdx.x & 63;
  const int j = lane % LPT;                            // 32-value chunk of the token
  // token indices and offsets are 32-bit: the host keeps n * head_dim / 2
  // below 2^27, so n < 2^23 and the GRP * n logits stay below 2^31 bytes
  const int n = (int)n64;
  // query slices: q[l][h*GRP + g][32 j .. 32 j + 32) as 16 bf16 pairs per head
  uint32_t qv[GRP][16];
#pragma unroll
  for (int g = 0; g < GRP; ++g) {
    const u32x4* qp = (const u32x4*)(q + ((int64_t)l * q_heads + h * GRP + g) * (LPT * 16) + j * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 w = qp[i];
      qv[g][4 * i] = w.x; qv[g][4 * i + 1] = w.y; qv[g][4 * i + 2] = w.z; qv[g][4 * i + 3] = w.w;
    }
  }
  const float gk = c.k_g[l * H + h];
  const int64_t row0 = ((int64_t)l * H + h) * c.capacity;
  // buffer resources over tokens [0, n) of this (layer, head), and over the
  // GRP logit rows of its query heads: loads past n read zeros, stores
  // steered past the extent write nothing, with no branch
  const __amdgpu_buffer_rsrc_t kc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.k + row0 * LPT * 16), 0, n * LPT * 16, kBufferWord3);          // 16 code bytes per lane
  const __amdgpu_buffer_rsrc_t ks = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(c.k_sf + row0 * LPT * 2), 0, n * LPT * 2, kBufferWord3);         // 2 scale bytes per lane
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(logits + ((int64_t)l * q_heads + h * GRP) * n64), 0, GRP * n * 4, kBufferWord3);
  const int tok_step = (int)gridDim.x * (kThreads / 64) * TPW;
  const int t_lane = lane / LPT;
  // U token groups per trip (independent dot chains); two register sets
  // alternate, so the next trip's codes and scales are in flight while this
  // trip is contracted
  int t = ((int)blockIdx.x * (kThreads / 64) + wave_id()) * TPW + t_lane;
  auto load = [&](int t0, u32x4 (&cw)[U], uint32_t (&sw)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tu = t0 + u * tok_step;
      const uint32_t e = tu < n ? (uint32_t)(tu * LPT + j) : 0x08000000u;     // past the extent: zeros
      cw[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kc, (int)(e * 16u), 0, kStreamLoad));
      sw[u] = __builtin_amdgcn_raw_buffer_load_b16(ks, (int)(e * 2u), 0, kStreamLoad);
    }
  };
  auto contract = [&](int t0, const u32x4 (&cw)[U], const uint32_t (&sw)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // scales from their E4M3 bytes (exact hardware decode)
      const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sw[u], 0), s1 = __builtin_amdgcn_cvt_f32_fp8((int)sw[u], 1);
      bf16x2 kp[16];
      kp[0] = kpair<0>(cw[u].x); kp[1] = kpair<1>(cw[u].x); kp[2] = kpair<2>(cw[u].x); kp[3] = kpair<3>(cw[u].x);
      kp[4] = kpair<0>(cw[u].y); kp[5] = kpair<1>(cw[u].y); kp[6] = kpair<2>(cw[u].y); kp[7] = kpair<3>(cw[u].y);
      kp[8] = kpair<0>(cw[u].z); kp[9] = kpair<1>(cw[u].z); kp[10] = kpair<2>(cw[u].z); kp[11] = kpair<3>(cw[u].z);
      kp[12] = kpair<0>(cw[u].w); kp[13] = kpair<1>(cw[u].w); kp[14] = kpair<2>(cw[u].w); kp[15] = kpair<3>(cw[u].w);
      const int tu = t0 + u * tok_step;
      float tot[GRP];
#pragma unroll
      for (int g = 0; g < GRP; ++g) {
        float p0 = dot2_first(kp[0], __builtin_bit_cast(bf16x2, qv[g][0]));
        float p1 = dot2_first(kp[8], __builtin_bit_cast(bf16x2, qv[g][8]));
#pragma unroll
        for (int i = 1; i < 8; ++i) {
          p0 = __builtin_amdgcn_fdot2_f32_bf16(kp[i], __builtin_bit_cast(bf16x2, qv[g][i]), p0, false);
          p1 = __builtin_amdgcn_fdot2_f32_bf16(kp[8 + i], __builtin_bit_cast(bf16x2, qv[g][8 + i]), p1, false);
        }
        tot[g] = lane_group_sum<LPT>(__builtin_fmaf(p1, s1, p0 * s0));
      }
      // every lane of the token holds every head's total; lane j stores heads
      // j, j + LPT, ... (one store per head it owns).  A wave's store covers
      // 64-byte runs of several heads' rows, which L2 merges into whole lines:
      // non-temporal stores here ran 0.625 against 0.537 ms
      constexpr int kSPL = GRP >= LPT ? GRP / LPT : 1;
#pragma unroll
      for (int sidx = 0; sidx < kSPL; ++sidx) {
        const int g = sidx * LPT + j;
        float v = tot[0];
#pragma unroll
        for (int gg = 1; gg < GRP; ++gg) v = g == gg ? tot[gg] : v;
        const uint32_t off = (tu < n && g < GRP) ? (uint32_t)((g * n + tu) * 4) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v * gk), ro, (int)off, 0, 0);
      }
    }
  };
  u32x4 cwa[U], cwb[U];
  uint32_t swa[U], swb[U];
  const int trip = U * tok_step;
  load(t, cwa, swa);
  while (t - t_lane < n) {
    load(t + trip, cwb, swb);
    contract(t, cwa, swa);
    t += trip;
    if (t - t_lane >= n) break;
    load(t + trip, cwa, swa);
    contract(t, cwb, swb);
    t += trip;
  }
}

}  // namespace nvfp4

// ============================================================ host entry points
namespace {

using namespace nvfp4;

nvfp4_status check_desc(const nvfp4_kv_cache* c) {
  if (!c) return NVFP4_EINVAL;
  if (c->layers <= 0 || c->kv_heads <= 0 || c->head_dim <= 0 || c->capacity < 0) return NVFP4_EINVAL;
  if (c->head_dim % kBlock) return NVFP4_EINVAL;
  if (c->kv_heads > 65535 || c->layers > 32767) return NVFP4_EINVAL;
  if (!c->k || !c->v || !c->k_sf || !c->v_sf || !c->k_g || !c->v_g) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(c->k) || !nvfp4host::aligned16(c->v) || !nvfp4host::aligned16(c->k_sf) ||
      !nvfp4host::aligned16(c->v_sf))
    return NVFP4_EALIGN;
  if ((reinterpret_cast<uintptr_t>(c->k_g) & 3u) || (reinterpret_cast<uintptr_t>(c->v_g) & 3u)) return NVFP4_EALIGN;
  return NVFP4_OK;
}

int tiles_for(int64_t blocks, int64_t other_wgs) {
  const int64_t target = (int64_t)nvfp4host::num_cus() * 8;
  int64_t per = std::max<int64_t>(1, (target + other_wgs - 1) / other_wgs);
  const int64_t need = (blocks + kThreads - 1) / kThreads;
  return (int)std::max<int64_t>(1, std::min<int64_t>(std::min(per, need), 65535));
}

}  // namespace

extern "C" {

size_t nvfp4_kv_bytes(const nvfp4_kv_cache* c) {
  if (!c || c->layers <= 0 || c->kv_heads <= 0 || c->head_dim <= 0 || c->capacity < 0 || c->head_dim % kBlock)
    return 0;
  const size_t per_row = (size_t)c->head_dim / 2 + (size_t)c->head_dim / kBlock;   // 0.5625 B per value
  return 2 * (size_t)c->layers * (size_t)c->kv_heads * (size_t)c->capacity * per_row;
}

nvfp4_status nvfp4_kv_append(const nvfp4_kv_cache* c, int64_t start, int64_t n, const uint16_t* k_new,
                             const uint16_t* v_new, void* stream) {
  nvfp4_status st = check_desc(c);
  if (st) return st;
  if (start < 0 || n < 0 || start > c->capacity || n > c->capacity - start) return NVFP4_EINVAL;
  if (n == 0) return NVFP4_OK;
  if (!k_new || !v_new) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(k_new) || !nvfp4host::aligned16(v_new)) return NVFP4_EALIGN;
  const int R = c->head_dim / 8;
  if (n > INT32_MAX / R) return NVFP4_EINVAL;                      // 32-bit token index per lane
  if ((st = nvfp4host::check_device())) return st;
  const int64_t halves = n * R;
  const int tiles = (int)std::min<int64_t>((halves + kThreads * kKVU - 1) / (kThreads * kKVU), 65535);
  const bool pow2 = (R & (R - 1)) == 0;
  const int log2r = __builtin_ctz((unsigned)R);
  const dim3 grid(tiles, c->kv_heads, 2 * c->layers);
  if (pow2)
    kv_append_kernel<true><<<grid, kThreads, 0, (hipStream_t)stream>>>(*c, start, n, log2r, (const u32x4*)k_new,
                                                                      (const u32x4*)v_new);
  else
    kv_append_kernel<false><<<grid, kThreads, 0, (hipStream_t)stream>>>(*c, start, n, log2r, (const u32x4*)k_new,
                                                                       (const u32x4*)v_new);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

nvfp4_status nvfp4_kv_read(const nvfp4_kv_cache* c, int32_t layer0, int32_t nlayers, int64_t t0, int64_t n,
                           uint16_t* k_out, uint16_t* v_out, void* stream) {
  nvfp4_status st = check_desc(c);
  if (st) return st;
  if (layer0 < 0 || nlayers < 0 || layer0 > c->layers || nlayers > c->layers - layer0) return NVFP4_EINVAL;
  if (t0 < 0 || n < 0 || t0 > c->capacity || n > c->capacity - t0) return NVFP4_EINVAL;
  if (n == 0 || nlayers == 0 || (!k_out && !v_out)) return NVFP4_OK;
  if (!nvfp4host::aligned16(k_out) || !nvfp4host::aligned16(v_out)) return NVFP4_EALIGN;
  if ((st = nvfp4host::check_device())) return st;
  const int64_t halves = n * (c->head_dim / 8);
  // one pass: each lane takes its kKVReadU half blocks once, so the workgroups
  // in flight write close together (0.566 -> 0.494 ms for 4 layers x 131072
  // tokens against ~8 resident workgroups per CU striding over every slice)
  const int tiles = (int)std::max<int64_t>(
      1, std::min<int64_t>((halves + kThreads * kKVReadU - 1) / (kThreads * kKVReadU), (int64_t)1 << 30));
  kv_read_kernel<<<dim3(tiles, c->kv_heads, 2 * nlayers), kThreads, 0, (hipStream_t)stream>>>(
      *c, layer0, t0, n, (u32x4*)k_out, (u32x4*)v_out);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

nvfp4_status nvfp4_kv_decode_qk(const nvfp4_kv_cache* c, const uint16_t* q, int32_t q_heads, int64_t n,
                                float* logits, void* stream) {
  nvfp4_status st = check_desc(c);
  if (st) return st;
  if (q_heads <= 0 || q_heads % c->kv_heads) return NVFP4_EINVAL;
  const int grp = q_heads / c->kv_heads;
  const int bpr = c->head_dim / kBlock;
  if (grp > 16 || (int64_t)grp * c->head_dim > kQKMaxLds) return NVFP4_ENOTSUP;
  if (bpr > 64 || (bpr & (bpr - 1))) return NVFP4_ENOTSUP;
  if (n < 0 || n > c->capacity) return NVFP4_EINVAL;
  if (n == 0) return NVFP4_OK;
  if (!q || !logits) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(q) || !nvfp4host::aligned16(logits)) return NVFP4_EALIGN;
  if ((st = nvfp4host::check_device())) return st;
  const int lpt = c->head_dim / 32;
  // 32-bit buffer offsets: n * head_dim / 2 code bytes per (layer, head)
  if (c->head_dim % 32 == 0 && (lpt == 1 || lpt == 2 || lpt == 4 || lpt == 8) &&
      (grp == 1 || grp == 2 || grp == 4 || grp == 8) && n * (c->head_dim / 2) < (INT64_C(1) << 27)) {
    const int64_t tpb = (kThreads / 64) * (64 / lpt);             // tokens per workgroup pass
    const int64_t need = (n + tpb - 1) / tpb;
    const int64_t per = std::max<int64_t>(1, (int64_t)nvfp4host::num_cus() * 8 / ((int64_t)c->kv_heads * c->layers));
    const int tiles = (int)std::max<int64_t>(1, std::min<int64_t>(need, std::min<int64_t>(per, 65535)));
    const dim3 grid(tiles, c->kv_heads, c->layers);
    hipStream_t st = (hipStream_t)stream;
    const uint32_t* qa = (const uint32_t*)q;
#define NVFP4_QK(L, G) kv_qk_kernel<L, G><<<grid, kThreads, 0, st>>>(*c, qa, q_heads, n, logits)
    switch (lpt * 16 + grp) {
      case 1 * 16 + 1: NVFP4_QK(1, 1); break;
      case 1 * 16 + 2: NVFP4_QK(1, 2); break;
      case 1 * 16 + 4: NVFP4_QK(1, 4); break;
      case 1 * 16 + 8: NVFP4_QK(1, 8); break;
      case 2 * 16 + 1: NVFP4_QK(2, 1); break;
      case 2 * 16 + 2: NVFP4_QK(2, 2); break;
      case 2 * 16 + 4: NVFP4_QK(2, 4); break;
      case 2 * 16 + 8: NVFP4_QK(2, 8); break;
      case 4 * 16 + 1: NVFP4_QK(4, 1); break;
      case 4 * 16 + 2: NVFP4_QK(4, 2); break;
      case 4 * 16 + 4: NVFP4_QK(4, 4); break;
      case 4 * 16 + 8: NVFP4_QK(4, 8); break;
      case 8 * 16 + 1: NVFP4_QK(8, 1); break;
      case 8 * 16 + 2: NVFP4_QK(8, 2); break;
      case 8 * 16 + 4: NVFP4_QK(8, 4); break;
      default: NVFP4_QK(8, 8); break;
    }
#undef NVFP4_QK
    NVFP4_LAUNCH_CHECK();
    return NVFP4_OK;
  }
  const int64_t tokens_per_iter = kThreads / bpr;
  const int64_t need = (n + tokens_per_iter - 1) / tokens_per_iter;
  const int tiles = (int)std::max<int64_t>(
      1, std::min<int64_t>(need, std::max<int64_t>(1, (int64_t)nvfp4host::num_cus() * 8 /
                                                           ((int64_t)c->kv_heads * c->layers))));
  kv_decode_qk_kernel<<<dim3(tiles, c->kv_heads, c->layers), kThreads, 0, (hipStream_t)stream>>>(*c, q, q_heads, n,
                                                                                                  logits);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

}  // extern "C"
