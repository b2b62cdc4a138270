// Quantize / dequantize kernels and their C-ABI entry points.
//
// Two-level microscaling (axbrief.com, "NVFP4: how NVIDIA pre-trained a 12B
// model on 10 trillion tokens", section "E2M1 format and two-level scaling"):
// pass 1 reduces the tensor amax (the FP32 tensor scale sets the overall
// range), pass 2 derives each 16-value block's E4M3 scale from its amax and
// rounds every element onto the E2M1 grid, packing two codes per byte.
// Dequantization restores values from the scales (omidsaffari.com, "LLM
// quantization guide", section "What is LLM quantization").
//
// Memory layout per tensor: a flat run of 16-value blocks (rows never split a
// block because cols % 16 == 0): x block i at 32*i bytes, codes at 8*i,
// scale byte at i.  One thread handles one block per iteration; consecutive
// lanes take consecutive blocks, so every wave reads 2 KiB and writes 512 B
// of codes contiguously.
#include <algorithm>

#include "common.hpp"

namespace nvfp4 {

// ------------------------------------------------------------ pass 1: amax
// grid (P, batch): workgroup p of tensor t reduces a strided share of the
// tensor's 16-byte vectors and writes one partial maximum (bf16 magnitude
// bits) to partial[t*P + p].  No atomics, no zero-fill: pass 2 reduces the P
// partials itself.
__global__ void __launch_bounds__(kThreads) amax_partial_kernel(const u32x4* __restrict__ x, int64_t vec_per_tensor,
                                                                uint32_t* __restrict__ partial) {
  const int t = blockIdx.y;
  const u32x4* xt = x + (int64_t)t * vec_per_tensor;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t m0 = 0, m1 = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < vec_per_tensor; i += 4 * stride) {
    const u32x4 a = xt[i];
    const u32x4 b = xt[i + stride];
    const u32x4 c = xt[i + 2 * stride];
    const u32x4 d = xt[i + 3 * stride];
    m0 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m0, a.x), a.y), a.z), a.w);
    m1 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m1, b.x), b.y), b.z), b.w);
    m0 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m0, c.x), c.y), c.z), c.w);
    m1 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m1, d.x), d.y), d.z), d.w);
  }
  for (; i < vec_per_tensor; i += stride) {
    const u32x4 a = xt[i];
    m0 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m0, a.x), a.y), a.z), a.w);
  }
  uint32_t m = halves_max(pk_absmax(m0, m1));
  m = wave_max_u32(m);
  __shared__ uint32_t red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = r > red[w] ? r : red[w];
    partial[(int64_t)t * gridDim.x + blockIdx.x] = r;
  }
}

// ------------------------------------------------------------ pass 2: encode
// Shared prologue: the tensor scale g, d6 = RN32(6g), r6 = RN32(1/d6) and the
// 127-entry encode table in LDS.
struct TensorScales {
  float g, d6, r6;
  bool zero_all, exact_all;
};

__device__ __forceinline__ TensorScales make_scales(float g) {
  TensorScales ts;
  ts.g = g;
  ts.d6 = 6.0f * g;
  ts.zero_all = ts.d6 == 0.0f;
  ts.exact_all = !(ts.d6 >= 0x1p-125f && ts.d6 <= 0x1p125f);
  ts.r6 = (ts.zero_all || ts.exact_all) ? 0.0f : 1.0f / ts.d6;
  return ts;
}

__device__ __forceinline__ void build_table(Entry* table, float g) {
  for (uint32_t j = threadIdx.x; j < 127u; j += kThreads) table[j] = build_entry(j, g);
}

__device__ __forceinline__ void load_block(const u32x4* __restrict__ xb, uint32_t (&w)[8]) {
  const u32x4 a = xb[0];
  const u32x4 b = xb[1];
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

__device__ __forceinline__ void encode_store(const uint32_t (&w)[8], const TensorScales& ts, const Entry* table,
                                             u32x2* __restrict__ qb, uint8_t* __restrict__ sb) {
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = pk_absmax(am, w[i]);
  const uint32_t sbyte = block_scale_byte(halves_max(am), ts.d6, ts.r6, ts.exact_all, ts.zero_all);
  const Entry en = table[sbyte];
  uint32_t c0, c1;
  encode_block(w, en, sbyte, ts.g, c0, c1);
  *qb = u32x2{c0, c1};
  *sb = (uint8_t)sbyte;
}

// grid (P, batch).  kFromPartials: g = RN32(amax/2688) from pass-1 partials;
// otherwise g is read from gin[t] (quantize_with_scale).
template <bool kFromPartials>
__global__ void __launch_bounds__(kThreads) encode_kernel(const u32x4* __restrict__ x, int64_t blk_per_tensor,
                                                          const uint32_t* __restrict__ partial, int npartial,
                                                          const float* __restrict__ gin, float* __restrict__ gout,
                                                          u32x2* __restrict__ q, uint8_t* __restrict__ sf) {
  const int t = blockIdx.y;
  __shared__ Entry table[128];
  __shared__ uint32_t red[kThreads / 64];
  float g;
  if (kFromPartials) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += kThreads) {
      const uint32_t v = partial[(int64_t)t * npartial + i];
      m = m > v ? m : v;
    }
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t amax_bits = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) amax_bits = amax_bits > red[w] ? amax_bits : red[w];
    g = __uint_as_float(amax_bits << 16) / kGlobalDiv;
    if (blockIdx.x == 0 && threadIdx.x == 0) gout[t] = g;
  } else {
    g = gin[t];
  }
  const TensorScales ts = make_scales(g);
  build_table(table, g);
  __syncthreads();

  const int64_t base = (int64_t)t * blk_per_tensor;
  const u32x4* xt = x + 2 * base;
  u32x2* qt = q + base;
  uint8_t* st = sf + base;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + stride < blk_per_tensor; i += 2 * stride) {
    uint32_t w0[8], w1[8];
    load_block(xt + 2 * i, w0);
    load_block(xt + 2 * (i + stride), w1);
    encode_store(w0, ts, table, qt + i, st + i);
    encode_store(w1, ts, table, qt + i + stride, st + i + stride);
  }
  for (; i < blk_per_tensor; i += stride) {
    uint32_t w0[8];
    load_block(xt + 2 * i, w0);
    encode_store(w0, ts, table, qt + i, st + i);
  }
}

// ------------------------------------------------------------ dequantize
// Per block: 8 code bytes + 1 scale byte -> 16 bf16.  v = RN32((E2M1*s)*g):
// the hardware decode gives the exact signed E2M1 value, E2M1*s is exact in
// f32, one rounding for *g, then RNE to bf16.
__device__ __forceinline__ uint32_t dequant_pair(uint32_t codes, int sel, float s, float g) {
  f32x2 f;
  switch (sel) {
    case 0: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0); break;
    case 1: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1); break;
    case 2: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2); break;
    default: f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3); break;
  }
  const float a = (f.x * s) * g;
  const float b = (f.y * s) * g;
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

__device__ __forceinline__ void dequant_block(u32x2 c, uint8_t sbyte, float g, u32x4* __restrict__ yb) {
  const float s = e4m3_value(sbyte);
  u32x4 o0, o1;
  o0.x = dequant_pair(c.x, 0, s, g);
  o0.y = dequant_pair(c.x, 1, s, g);
  o0.z = dequant_pair(c.x, 2, s, g);
  o0.w = dequant_pair(c.x, 3, s, g);
  o1.x = dequant_pair(c.y, 0, s, g);
  o1.y = dequant_pair(c.y, 1, s, g);
  o1.z = dequant_pair(c.y, 2, s, g);
  o1.w = dequant_pair(c.y, 3, s, g);
  yb[0] = o0;
  yb[1] = o1;
}

__global__ void __launch_bounds__(kThreads) dequant_kernel(const u32x2* __restrict__ q, const uint8_t* __restrict__ sf,
                                                           const float* __restrict__ gin, int64_t blk_per_tensor,
                                                           u32x4* __restrict__ y) {
  const int t = blockIdx.y;
  const float g = gin[t];
  const int64_t base = (int64_t)t * blk_per_tensor;
  const u32x2* qt = q + base;
  const uint8_t* st = sf + base;
  u32x4* yt = y + 2 * base;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + stride < blk_per_tensor; i += 2 * stride) {
    const u32x2 c0 = qt[i];
    const u32x2 c1 = qt[i + stride];
    const uint8_t s0 = st[i], s1 = st[i + stride];
    dequant_block(c0, s0, g, yt + 2 * i);
    dequant_block(c1, s1, g, yt + 2 * (i + stride));
  }
  for (; i < blk_per_tensor; i += stride) dequant_block(qt[i], st[i], g, yt + 2 * i);
}

}  // namespace nvfp4

// ============================================================ host entry points
namespace {

using namespace nvfp4;

// Workgroups per tensor for a streaming launch: enough to fill the GPU
// (~8 workgroups per CU overall) but at least 16 blocks per thread.
int wgs_per_tensor(int64_t batch, int64_t blk_per_tensor) {
  const int64_t target = (int64_t)nvfp4host::num_cus() * 8;
  int64_t per = (target + batch - 1) / batch;
  const int64_t need = (blk_per_tensor + (int64_t)kThreads * 16 - 1) / ((int64_t)kThreads * 16);
  per = std::min(per, need);
  per = std::max<int64_t>(per, 1);
  return (int)std::min<int64_t>(per, 65535);
}

constexpr int kMaxPartials = 2048;

int amax_wgs_per_tensor(int64_t batch, int64_t vec_per_tensor) {
  const int64_t target = (int64_t)nvfp4host::num_cus() * 8;
  int64_t per = (target + batch - 1) / batch;
  const int64_t need = (vec_per_tensor + (int64_t)kThreads * 16 - 1) / ((int64_t)kThreads * 16);
  per = std::min<int64_t>(std::min(per, need), kMaxPartials);
  return (int)std::max<int64_t>(per, 1);
}

nvfp4_status check_shape(int64_t batch, int64_t rows, int64_t cols) {
  if (batch < 0 || rows < 0 || cols < 0 || cols % kBlock) return NVFP4_EINVAL;
  if (batch > 65535) return NVFP4_EINVAL;                        // grid.y
  if (rows > 0 && cols > 0 && rows > (INT64_C(1) << 58) / cols) return NVFP4_EINVAL;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

size_t nvfp4_quantize_workspace_bytes(int64_t batch, int64_t rows, int64_t cols) {
  if (batch <= 0 || rows < 0 || cols < 0) return 0;
  (void)rows;
  (void)cols;
  // per-tensor partial maxima of pass 1, plus one 256-byte header reserved
  // for the persistent launch's counters.
  return 256 + (size_t)batch * kMaxPartials * sizeof(uint32_t);
}

nvfp4_status nvfp4_quantize(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sf,
                            float* g, void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  nvfp4_status st = check_shape(batch, rows, cols);
  if (st) return st;
  if (flags != NVFP4_TWO_KERNEL) return NVFP4_ENOTSUP;   // the persistent launch is not built yet
  if (batch == 0) return NVFP4_OK;
  if (!g) return NVFP4_EINVAL;
  const int64_t n = rows * cols;
  if (n > 0 && (!x || !q || !sf)) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(x) || !nvfp4host::aligned16(q) || !nvfp4host::aligned16(sf) || !nvfp4host::aligned16(g))
    return NVFP4_EALIGN;
  if (!workspace || workspace_bytes < nvfp4_quantize_workspace_bytes(batch, rows, cols)) return NVFP4_EWORKSPACE;
  if (!nvfp4host::aligned16(workspace)) return NVFP4_EALIGN;
  if ((st = nvfp4host::check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* partial = (uint32_t*)((char*)workspace + 256);
  const int64_t vec = n / 8, blk = n / kBlock;
  const int p1 = amax_wgs_per_tensor(batch, vec);
  amax_partial_kernel<<<dim3(p1, (unsigned)batch), kThreads, 0, s>>>((const u32x4*)x, vec, partial);
  NVFP4_LAUNCH_CHECK();
  const int p2 = wgs_per_tensor(batch, blk);
  encode_kernel<true><<<dim3(p2, (unsigned)batch), kThreads, 0, s>>>((const u32x4*)x, blk, partial, p1, nullptr, g,
                                                                      (u32x2*)q, sf);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

nvfp4_status nvfp4_quantize_with_scale(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, const float* g,
                                       uint8_t* q, uint8_t* sf, void* stream) {
  nvfp4_status st = check_shape(batch, rows, cols);
  if (st) return st;
  const int64_t n = rows * cols;
  if (batch == 0 || n == 0) return NVFP4_OK;
  if (!x || !q || !sf || !g) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(x) || !nvfp4host::aligned16(q) || !nvfp4host::aligned16(sf)) return NVFP4_EALIGN;
  if ((reinterpret_cast<uintptr_t>(g) & 3u) != 0) return NVFP4_EALIGN;
  if ((st = nvfp4host::check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  const int64_t blk = n / kBlock;
  const int p2 = wgs_per_tensor(batch, blk);
  encode_kernel<false><<<dim3(p2, (unsigned)batch), kThreads, 0, s>>>((const u32x4*)x, blk, nullptr, 0, g, nullptr,
                                                                       (u32x2*)q, sf);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

nvfp4_status nvfp4_dequantize(const uint8_t* q, const uint8_t* sf, const float* g, int64_t batch, int64_t rows,
                              int64_t cols, uint16_t* y, void* stream) {
  nvfp4_status st = check_shape(batch, rows, cols);
  if (st) return st;
  const int64_t n = rows * cols;
  if (batch == 0 || n == 0) return NVFP4_OK;
  if (!q || !sf || !g || !y) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(q) || !nvfp4host::aligned16(sf) || !nvfp4host::aligned16(y)) return NVFP4_EALIGN;
  if ((reinterpret_cast<uintptr_t>(g) & 3u) != 0) return NVFP4_EALIGN;
  if ((st = nvfp4host::check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  const int64_t blk = n / kBlock;
  const int p = wgs_per_tensor(batch, blk);
  dequant_kernel<<<dim3(p, (unsigned)batch), kThreads, 0, s>>>((const u32x2*)q, sf, g, blk, (u32x4*)y);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

}  // extern "C"
