// Block-scaled NVFP4 x NVFP4 GEMM on gfx950 bf16 MFMA.
//
// NVFP4 serves both weights and activations of MoE expert linears (iwan.kr,
// "NVIDIA shrank GLM-5.2 to 4 bits", section 1); the low-bit operands are
// restored inside the compute kernel instead of being expanded in global
// memory (omidsaffari.com, "LLM quantization guide", section "memory, speed
// and quality").  gfx950 has no MFMA that consumes E4M3-per-16 block scales,
// so each 16-value block is dequantized EXACTLY to bf16 (E2M1 * s has at most
// 6 significant bits and lies in [2^-10, 2688]) in LDS, contracted on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation, and the two FP32 tensor
// scales are applied once in the epilogue.
//
// C[m][n] = gA * gB * sum_k deq(A)[m][k] * deq(B)[n][k]   (both K-major)
#include <algorithm>

#include "common.hpp"

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int GLDK = GBK + 8;          // LDS row stride in bf16 (pads away bank conflicts)

// Dequantizes one 16-value block (8 code bytes, scale byte) into 16 bf16 at dst.
__device__ __forceinline__ void deq16_to_lds(u32x2 c, uint32_t sbyte, __bf16* dst) {
  const float s = e4m3_value(sbyte);
  bf16x8 lo, hi;
  f32x2 f;
  f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 0); lo[0] = (__bf16)(f.x * s); lo[1] = (__bf16)(f.y * s);
  f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 1); lo[2] = (__bf16)(f.x * s); lo[3] = (__bf16)(f.y * s);
  f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 2); lo[4] = (__bf16)(f.x * s); lo[5] = (__bf16)(f.y * s);
  f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 3); lo[6] = (__bf16)(f.x * s); lo[7] = (__bf16)(f.y * s);
  f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 0); hi[0] = (__bf16)(f.x * s); hi[1] = (__bf16)(f.y * s);
  f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 1); hi[2] = (__bf16)(f.x * s); hi[3] = (__bf16)(f.y * s);
  f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 2); hi[4] = (__bf16)(f.x * s); hi[5] = (__bf16)(f.y * s);
  f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 3); hi[6] = (__bf16)(f.x * s); hi[7] = (__bf16)(f.y * s);
  *(bf16x8*)dst = lo;
  *(bf16x8*)(dst + 8) = hi;
}

// Stages a GBM x GBK (or GBN x GBK) tile: 512 blocks of 16 values, 2 per thread.
__device__ __forceinline__ void stage_tile(const uint8_t* __restrict__ q, const uint8_t* __restrict__ sf, int64_t rows,
                                           int64_t K, int64_t r0, int64_t k0, __bf16 (*tile)[GLDK]) {
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int idx = threadIdx.x + it * kThreads;   // 0..511
    const int r = idx >> 2, kb = idx & 3;
    const int64_t gr = r0 + r, gk = k0 + 16 * kb;
    u32x2 c = {0u, 0u};
    uint32_t sb = 0;
    if (gr < rows && gk < K) {
      c = *(const u32x2*)(q + gr * (K / 2) + gk / 2);
      sb = sf[gr * (K / 16) + gk / 16];
    }
    deq16_to_lds(c, sb, &tile[r][16 * kb]);
  }
}

__global__ void __launch_bounds__(kThreads) gemm_lds_kernel(const uint8_t* __restrict__ aq,
                                                            const uint8_t* __restrict__ asf,
                                                            const float* __restrict__ ag,
                                                            const uint8_t* __restrict__ bq,
                                                            const uint8_t* __restrict__ bsf,
                                                            const float* __restrict__ bg, int64_t M, int64_t N,
                                                            int64_t K, float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) __bf16 As[GBM][GLDK];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[GBN][GLDK];
  const int64_t m0 = (int64_t)blockIdx.y * GBM, n0 = (int64_t)blockIdx.x * GBN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;       // 2 x 2 waves, 64 x 64 each
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  for (int64_t k0 = 0; k0 < K; k0 += GBK) {
    stage_tile(aq, asf, M, K, m0, k0, As);
    stage_tile(bq, bsf, N, K, n0, k0, Bs);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GBK; kk += 16) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *(const bf16x8*)&As[wm * 64 + i * 32 + (lane & 31)][kk + 8 * (lane >> 5)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8*)&Bs[wn * 64 + j * 32 + (lane & 31)][kk + 8 * (lane >> 5)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  const float gab = ag[0] * bg[0];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < M && col < N) C[row * N + col] = acc[i][j][e] * gab;
      }
}

}  // namespace nvfp4

extern "C" nvfp4_status nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_sf, const float* a_g, const uint8_t* b_q,
                                   const uint8_t* b_sf, const float* b_g, int64_t M, int64_t N, int64_t K, float* c,
                                   void* stream) {
  using namespace nvfp4;
  if (M < 0 || N < 0 || K < 0 || K % kBlock) return NVFP4_EINVAL;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a_g || !b_g || !c) return NVFP4_EINVAL;
  if (K > 0 && (!a_q || !a_sf || !b_q || !b_sf)) return NVFP4_EINVAL;
  if ((M + GBM - 1) / GBM > 65535 || (N + GBN - 1) / GBN > 2147483647LL) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(a_q) || !nvfp4host::aligned16(b_q) || !nvfp4host::aligned16(c)) return NVFP4_EALIGN;
  if ((reinterpret_cast<uintptr_t>(a_g) & 3u) || (reinterpret_cast<uintptr_t>(b_g) & 3u)) return NVFP4_EALIGN;
  nvfp4_status st = nvfp4host::check_device();
  if (st) return st;
  dim3 grid((unsigned)((N + GBN - 1) / GBN), (unsigned)((M + GBM - 1) / GBM));
  gemm_lds_kernel<<<grid, kThreads, 0, (hipStream_t)stream>>>(a_q, a_sf, a_g, b_q, b_sf, b_g, M, N, K, c);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}
