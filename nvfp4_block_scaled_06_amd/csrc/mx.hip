// MXFP4: the earlier microscaling format, 32 E2M1 values sharing one
// power-of-two (E8M0) scale, no tensor scale, about 4.25 bits per value
// (iwan.kr, "NVIDIA shrank GLM-5.2 to 4 bits", section 3 "Terminology";
// axbrief.com, "NVFP4: how NVIDIA pre-trained a 12B model on 10 trillion
// tokens", section "36% token efficiency and Blackwell speed"; theddari.com,
// "What is FP4 quantization? KV cache in 4 bits", format comparison table).
//
// The pages leave the exponent rule open; this follows the published
// Microscaling definition of the format:
//   X = floor(log2(block amax)) - 2, clamped to [-127, 127] (an all-zero
//       block takes -127); scale byte X + 127; 2 is the exponent of 6, the
//       largest E2M1 value
//   code = sign | E2M1_RNE_SAT(|x| / 2^X);  dequant bf16(E2M1 * 2^X)
// For bf16 input the exponent is integer work: with e the biased exponent
// of the block amax, the scale byte is max(e - 2, 0), and |x| / 2^X is the
// exact product |x| * 2^(127 - byte).
//
// gfx950 contracts MXFP4 natively: v_mfma_scale_f32_32x32x64_f8f6f4 with
// fp4 operands takes, per lane, 32 consecutive K values of one row (16
// bytes, element 2j in the low nibble of byte j, as stored) and that
// block's E8M0 byte, so the GEMM feeds raw codes and scale bytes from LDS to
// the matrix cores with no dequantization at all.
#include <algorithm>

#include "common.hpp"

namespace nvfp4 {

constexpr int kMxBlock = 32;

// ------------------------------------------------------------ quantize
// Each lane takes a quarter block (8 values, 16 bytes of bf16); the four
// lanes of a DPP quad hold one block and exchange partial maxima.
__device__ __forceinline__ uint32_t quad_max(uint32_t m) {
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);   // lane ^ 1
  m = m > o ? m : o;
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false);            // lane ^ 2
  return m > o ? m : o;
}

// Scale byte from the block amax's bf16 magnitude bits.
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
  const uint32_t e = amax_bits >> 7;                 // biased exponent (sign bit is 0)
  return e > 2u ? e - 2u : 0u;
}

__device__ __forceinline__ uint32_t mx_encode_quarter(const u32x4 w, float inv) {
  uint32_t c = fp4_pair<0>(0u, bf16_lo(w.x) * inv, bf16_hi(w.x) * inv);
  c = fp4_pair<1>(c, bf16_lo(w.y) * inv, bf16_hi(w.y) * inv);
  c = fp4_pair<2>(c, bf16_lo(w.z) * inv, bf16_hi(w.z) * inv);
  return fp4_pair<3>(c, bf16_lo(w.w) * inv, bf16_hi(w.w) * inv);
}

constexpr int kMxU = 4;   // quarter blocks per lane per loop trip

// nq quarter blocks (a multiple of 4, so a quad is wholly in or out of range).
__global__ void __launch_bounds__(kThreads) mx_quantize_kernel(const u32x4* __restrict__ x, int64_t nq,
                                                               uint32_t* __restrict__ q, uint8_t* __restrict__ sf) {
  const int lane = threadIdx.x & 63;
  const int64_t step = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kMxU - 1) * step < nq; i += kMxU * step) {
    u32x4 v[kMxU];
#pragma unroll
    for (int u = 0; u < kMxU; ++u) v[u] = __builtin_nontemporal_load(x + i + u * step);
#pragma unroll
    for (int u = 0; u < kMxU; ++u) {
      const uint32_t sbyte = mx_scale_byte(quad_max(half_absmax_bits(v[u])));
      const float inv = __uint_as_float((254u - sbyte) << 23);      // 2^(127 - byte) = 2^-X
      __builtin_nontemporal_store(mx_encode_quarter(v[u], inv), q + i + u * step);
      if ((lane & 3) == 0) sf[(i + u * step) >> 2] = (uint8_t)sbyte;
    }
  }
  for (; i < nq; i += step) {
    const u32x4 v = x[i];
    const uint32_t sbyte = mx_scale_byte(quad_max(half_absmax_bits(v)));
    q[i] = mx_encode_quarter(v, __uint_as_float((254u - sbyte) << 23));
    if ((lane & 3) == 0) sf[i >> 2] = (uint8_t)sbyte;
  }
}

// ------------------------------------------------------------ dequantize
// 2^(byte - 127) as fp32 (byte 0 is the subnormal 2^-127), NaN for 255.
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return b == 0u ? __uint_as_float(0x00400000u) : b == 255u ? __uint_as_float(0x7fc00000u) : __uint_as_float(b << 23);
}

__device__ __forceinline__ uint32_t mx_deq_pair_bits(f32x2 f, float sc) {
  const __bf16 ha = (__bf16)(f.x * sc), hb = (__bf16)(f.y * sc);
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

__device__ __forceinline__ u32x4 mx_dequant_quarter(uint32_t codes, float sc) {
  u32x4 o;
  o.x = mx_deq_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0), sc);
  o.y = mx_deq_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1), sc);
  o.z = mx_deq_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2), sc);
  o.w = mx_deq_pair_bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3), sc);
  return o;
}

// bf16 output stored non-temporal, as in the NVFP4 dequantize.
__global__ void __launch_bounds__(kThreads) mx_dequant_kernel(const uint32_t* __restrict__ q,
                                                              const uint8_t* __restrict__ sf, int64_t nq,
                                                              u32x4* __restrict__ y) {
  const int64_t step = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kMxU - 1) * step < nq; i += kMxU * step) {
    uint32_t c[kMxU];
    uint32_t s[kMxU];
#pragma unroll
    for (int u = 0; u < kMxU; ++u) {
      c[u] = __builtin_nontemporal_load(q + i + u * step);
      s[u] = sf[(i + u * step) >> 2];
    }
#pragma unroll
    for (int u = 0; u < kMxU; ++u)
      __builtin_nontemporal_store(mx_dequant_quarter(c[u], e8m0_value(s[u])), y + i + u * step);
  }
  for (; i < nq; i += step) __builtin_nontemporal_store(mx_dequant_quarter(q[i], e8m0_value(sf[i >> 2])), y + i);
}

// ------------------------------------------------------------ GEMM
//   C[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k]      (both K-major MXFP4)
//
// 256 x 256 output per workgroup, 4 waves of 128 x 128 (4 x 4 tiles of the
// 32 x 32 x 64 scaled MFMA, 256 fp32 accumulators per lane), K step 256
// values (128 code bytes and 8 scale bytes per row).  Each step's raw codes
// and scales are loaded into registers one step ahead and written to the
// other of two LDS buffers, one barrier per step.
//
// MFMA operand of tile row r in substep kk (64 values): lane l reads the 16
// code bytes of row r + l % 32 at byte 32 kk + 16 (l / 32), and the scale
// byte of block 2 kk + l / 32.  The loader stores, per row, the words
// W_h = bytes {h, 2 + h, 4 + h, 6 + h} of the row's 8 scale bytes (h = 0, 1),
// so lane l reads W_(l/32) once per step and substep kk selects byte kk
// (the instruction's op_sel).
constexpr int MTM = 256, MTN = 256;
constexpr int MTK = 256;                       // values per K step
constexpr int MROW = MTK / 2 + 16;             // LDS bytes per code row (16 bytes of padding)
constexpr int MThreads = 256;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct MxSmem {
  uint8_t a[2][MTM * MROW];
  uint8_t b[2][MTN * MROW];
  uint32_t as[2][MTM][2];
  uint32_t bs[2][MTN][2];
};

// One workgroup's rows [r0, r0 + 256) of an MXFP4 operand as buffer
// resources ending at the last row: rows past the matrix and blocks at or
// past K read zeros.
struct MxOperand {
  __amdgpu_buffer_rsrc_t q, s;
  uint32_t qrow, srow;                         // bytes per row: K/2, K/32
};

__device__ __forceinline__ MxOperand mx_operand(const uint8_t* q, const uint8_t* sf, int64_t r0, int64_t rows,
                                                int64_t K) {
  MxOperand o;
  const int64_t here = rows - r0 < MTM ? rows - r0 : MTM;
  o.qrow = (uint32_t)(K / 2);
  o.srow = (uint32_t)(K / 32);
  o.q = __builtin_amdgcn_make_buffer_rsrc((void*)(q + r0 * (K / 2)), 0, (int)(here * (K / 2)), kBufferWord3);
  o.s = __builtin_amdgcn_make_buffer_rsrc((void*)(sf + r0 * (K / 32)), 0, (int)(here * (K / 32)), kBufferWord3);
  return o;
}

constexpr uint32_t kMxOutside = 0x80000000u;   // past every extent (extents stay below 2^31)

// One thread's share of a K step of one operand: code chunk (tid % 8) (one
// block, 16 bytes) of rows tid / 8 + 32 j, j = 0..7, and the 8 scale bytes
// of row tid.
struct MxStep {
  u32x4 c[8];
  uint32_t w0, w1;                             // the row's W_0, W_1
};

// kAligned (K % 256 == 0): the caller only asks for steps inside K, so the
// loads carry no conditions; otherwise each block is checked on its own and
// blocks at or past K read as codes 0 with scale byte 0.
template <bool kAligned>
__device__ __forceinline__ MxStep mx_load_step(const MxOperand& o, int tid, int64_t K, int64_t k0) {
  MxStep st;
  const int chunk = tid & 7, rsub = tid >> 3;
  const uint32_t base = (uint32_t)rsub * o.qrow + (uint32_t)(k0 / 2) + 16u * chunk;
  const uint32_t cin = kAligned || k0 + 32 * chunk < K ? 0u : kMxOutside;   // this thread's block inside K
#pragma unroll
  for (int j = 0; j < 8; ++j)
    st.c[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(o.q, (int)((base + 32u * j * o.qrow) | cin), 0, 0));
  uint32_t lo, hi;
  const uint32_t so = (uint32_t)tid * o.srow + (uint32_t)(k0 / 32);
  if (kAligned) {
    const u32x2 s = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(o.s, (int)so, 0, 0));
    lo = s.x;
    hi = s.y;
  } else {
    lo = hi = 0u;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint32_t v = __builtin_amdgcn_raw_buffer_load_b8(o.s, (int)(k0 + 32 * b < K ? so + b : kMxOutside), 0, 0);
      if (b < 4) lo |= v << (8 * b);
      else hi |= v << (8 * (b - 4));
    }
  }
  // W_0 = bytes 0, 2, 4, 6 and W_1 = bytes 1, 3, 5, 7 of hi:lo
  st.w0 = __builtin_amdgcn_perm(hi, lo, 0x06040200u);
  st.w1 = __builtin_amdgcn_perm(hi, lo, 0x07050301u);
  return st;
}

__device__ __forceinline__ void mx_store_step(const MxStep& st, int tid, uint8_t* codes, uint32_t (*sc)[2]) {
  const int chunk = tid & 7, rsub = tid >> 3;
#pragma unroll
  for (int j = 0; j < 8; ++j) *(u32x4*)(codes + (rsub + 32 * j) * MROW + 16 * chunk) = st.c[j];
  sc[tid][0] = st.w0;
  sc[tid][1] = st.w1;
}

// Operand fragments of one substep: A tile rows i and B tile rows j.
struct MxFrag {
  i32x8 a[4], b[4];
};

__device__ __forceinline__ void mx_frag_load(MxFrag& f, const uint8_t* Acur, const uint8_t* Bcur, int kk) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = *(const u32x4*)(Acur + i * 32 * MROW + 32 * kk);
    f.a[i] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 v = *(const u32x4*)(Bcur + j * 32 * MROW + 32 * kk);
    f.b[j] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  }
}

// The 16 MFMAs of substep kk on f, while the fragments of substep kk + 1
// load from LDS into nf (kk < 3): one LDS read between every two MFMAs.
template <int kk>
__device__ __forceinline__ void mx_substep(f32x16 (&acc)[4][4], const MxFrag& f, MxFrag& nf, const uint8_t* Acur,
                                           const uint8_t* Bcur, const uint32_t (&sa)[4], const uint32_t (&sb)[4]) {
  __builtin_amdgcn_sched_barrier(0);
  if (kk < 3) mx_frag_load(nf, Acur, Bcur, kk + 1);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 4, 4, kk, (int)sa[i], kk,
                                                                  (int)sb[j]);
  if (kk < 3) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Writes a wave's 128 x 128 accumulators (rows wm*128.., columns wn*128..
// of the tile at (m0, n0)); C layout of the 32 x 32 MFMA: lane l, element e
// is row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32.
__device__ __forceinline__ void mx_epilogue(const f32x16 (&acc)[4][4], float* __restrict__ C, int64_t m0, int64_t n0,
                                            int64_t M, int64_t N, int wm, int wn, int lane) {
  float* Cw = C + (m0 + wm * 128 + 4 * (lane >> 5)) * N + n0 + wn * 128 + (lane & 31);
  if (m0 + MTM <= M && n0 + MTN <= N) {         // whole tile: no bounds checks
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) Cw[(i * 32 + 8 * (e >> 2) + (e & 3)) * N + j * 32] = acc[i][j][e];
  } else {
    const int64_t rlim = M - (m0 + wm * 128 + 4 * (lane >> 5)), clim = N - (n0 + wn * 128 + (lane & 31));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = i * 32 + 8 * (e >> 2) + (e & 3), cc = j * 32;
          if (r < rlim && cc < clim) Cw[r * N + cc] = acc[i][j][e];
        }
  }
}

template <bool kAligned>
__global__ void __launch_bounds__(MThreads) mx_gemm_kernel(const uint8_t* __restrict__ aq, const uint8_t* __restrict__ asf,
                                                           const uint8_t* __restrict__ bq, const uint8_t* __restrict__ bsf,
                                                           int64_t M, int64_t N, int64_t K, float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) MxSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tile = xcd_tile((int64_t)blockIdx.y * gridDim.x + blockIdx.x, (int64_t)gridDim.x * gridDim.y);
  const int64_t m0 = tile / gridDim.x * MTM, n0 = tile % gridDim.x * MTN;
  const MxOperand A = mx_operand(aq, asf, m0, M, K), B = mx_operand(bq, bsf, n0, N, K);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int64_t nk = (K + MTK - 1) / MTK;
  MxStep ra = mx_load_step<kAligned>(A, tid, K, 0), rb = mx_load_step<kAligned>(B, tid, K, 0);
  mx_store_step(ra, tid, sm.a[0], sm.as[0]);
  mx_store_step(rb, tid, sm.b[0], sm.bs[0]);
  __syncthreads();
  const int arow = wm * 128 + (lane & 31), brow = wn * 128 + (lane & 31), h = lane >> 5;
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    // the last step reloads itself (in range) into the unread buffer
    const int64_t knext = (kt + 1 < nk ? kt + 1 : kt) * MTK;
    ra = mx_load_step<kAligned>(A, tid, K, knext);
    rb = mx_load_step<kAligned>(B, tid, K, knext);
    const uint8_t* Acur = sm.a[buf] + arow * MROW + 16 * h;
    const uint8_t* Bcur = sm.b[buf] + brow * MROW + 16 * h;
    uint32_t sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = sm.as[buf][arow + 32 * i][h];
      sb[i] = sm.bs[buf][brow + 32 * i][h];
    }
    MxFrag f0, f1;
    mx_frag_load(f0, Acur, Bcur, 0);
    mx_substep<0>(acc, f0, f1, Acur, Bcur, sa, sb);
    mx_substep<1>(acc, f1, f0, Acur, Bcur, sa, sb);
    mx_substep<2>(acc, f0, f1, Acur, Bcur, sa, sb);
    mx_substep<3>(acc, f1, f0, Acur, Bcur, sa, sb);
    mx_store_step(ra, tid, sm.a[buf ^ 1], sm.as[buf ^ 1]);
    mx_store_step(rb, tid, sm.b[buf ^ 1], sm.bs[buf ^ 1]);
    __syncthreads();
  }
  mx_epilogue(acc, C, m0, n0, M, N, wm, wn, lane);
}


// ------------------------------------------------------------ GEMM, buffer-to-LDS loads
// The aligned GEMM (K % 256 == 0) moves each K step straight from HBM into
// LDS with buffer-to-LDS loads: no staging registers and no LDS writes by
// the waves, and step k+1 streams in while step k is contracted.
// A load instruction fills 1 KB of LDS, 16 bytes per lane in lane order, so
// code rows are stored unpadded (128 bytes) with their 16-byte chunks
// swizzled: chunk c of row r sits at position c ^ ((r >> 1) & 7).  The 16
// rows that 16 lanes of an MFMA fragment read then fall on distinct bank
// groups, and each lane loads the global chunk its LDS position holds.
// Scale bytes are stored raw (8 per row) and rearranged when read.
typedef __attribute__((address_space(3))) void mx_lds_t;

struct MxDmaSmem {
  uint8_t a[2][MTM * 128];
  uint8_t b[2][MTN * 128];
  uint32_t as[2][MTM][2];
  uint32_t bs[2][MTN][2];
};

// s_waitcnt vmcnt(0) with the other counters unconstrained; the compiler
// does not track the completion of buffer-to-LDS loads.
__device__ __forceinline__ void mx_wait_vm0() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
  __builtin_amdgcn_sched_barrier(0);
}

// 8 waves (two per SIMD), each a 128 x 64 eighth of the tile (4 x 2 MFMA
// tiles): a second wave per SIMD keeps the matrix cores busy while the
// other waits at the step barrier or on LDS.  Wave w loads code rows
// [32 w, 32 w + 32) of each operand (4 instructions of 8 rows) and their
// scale bytes (one instruction, 4 bytes per lane).
constexpr int MThreads8 = 512;

__device__ __forceinline__ void mx_dma_step8(const MxOperand& o, int wave, int lane, int64_t k0, uint8_t* codes,
                                             uint32_t (*sc)[2]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {                  // code rows [32 wave, 32 wave + 32)
    const int r = 32 * wave + 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.q, (mx_lds_t*)(codes + (32 * wave + 8 * j) * 128), 16,
                                             (uint32_t)r * o.qrow + (uint32_t)(k0 / 2) + 16u * c, 0, 0, 0);
  }
  const int r = 32 * wave + (lane >> 1);         // scale bytes of the same rows
  __builtin_amdgcn_raw_ptr_buffer_load_lds(o.s, (mx_lds_t*)&sc[32 * wave][0], 4,
                                           (uint32_t)r * o.srow + (uint32_t)(k0 / 32) + 4u * (lane & 1), 0, 0, 0);
}

struct MxFrag8 {
  i32x8 a[4], b[2];
};

__device__ __forceinline__ void mx_dma_frags8(MxFrag8& f, const uint8_t* Acur, const uint8_t* Bcur, int kk, int h,
                                              int sw) {
  const int pos = ((2 * kk + h) ^ sw) * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = *(const u32x4*)(Acur + i * 32 * 128 + pos);
    f.a[i] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const u32x4 v = *(const u32x4*)(Bcur + j * 32 * 128 + pos);
    f.b[j] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  }
}

template <int kk>
__device__ __forceinline__ void mx_dma_substep8(f32x16 (&acc)[4][2], const MxFrag8& f, MxFrag8& nf,
                                                const uint8_t* Acur, const uint8_t* Bcur, int h, int sw,
                                                const uint32_t (&sa)[4], const uint32_t (&sb)[2]) {
  __builtin_amdgcn_sched_barrier(0);
  if (kk < 3) mx_dma_frags8(nf, Acur, Bcur, kk + 1, h, sw);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 4, 4, kk, (int)sa[i], kk,
                                                                  (int)sb[j]);
  if (kk < 3) {
#pragma unroll
    for (int m = 0; m < 6; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

__global__ void __launch_bounds__(MThreads8) mx_gemm_dma8_kernel(const uint8_t* __restrict__ aq,
                                                                 const uint8_t* __restrict__ asf,
                                                                 const uint8_t* __restrict__ bq,
                                                                 const uint8_t* __restrict__ bsf, int64_t M,
                                                                 int64_t N, int64_t K, float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) MxDmaSmem sm;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wm = wave >> 2, wn = wave & 3;        // rows wm * 128 .., columns wn * 64 ..
  const int64_t tile = xcd_tile((int64_t)blockIdx.y * gridDim.x + blockIdx.x, (int64_t)gridDim.x * gridDim.y);
  const int64_t m0 = tile / gridDim.x * MTM, n0 = tile % gridDim.x * MTN;
  const MxOperand A = mx_operand(aq, asf, m0, M, K), B = mx_operand(bq, bsf, n0, N, K);

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int64_t nk = K / MTK;
  mx_dma_step8(A, wave, lane, 0, sm.a[0], sm.as[0]);
  mx_dma_step8(B, wave, lane, 0, sm.b[0], sm.bs[0]);
  mx_wait_vm0();
  __syncthreads();
  const int arow = wm * 128 + (lane & 31), brow = wn * 64 + (lane & 31), h = lane >> 5;
  const int sw = ((lane & 31) >> 1) & 7;
  const uint32_t sel = h ? 0x07050301u : 0x06040200u;
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < nk) {
      mx_dma_step8(A, wave, lane, (kt + 1) * MTK, sm.a[buf ^ 1], sm.as[buf ^ 1]);
      mx_dma_step8(B, wave, lane, (kt + 1) * MTK, sm.b[buf ^ 1], sm.bs[buf ^ 1]);
    }
    const uint8_t* Acur = sm.a[buf] + arow * 128;
    const uint8_t* Bcur = sm.b[buf] + brow * 128;
    uint32_t sa[4], sb[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t* ra = sm.as[buf][arow + 32 * i];
      sa[i] = __builtin_amdgcn_perm(ra[1], ra[0], sel);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t* rb = sm.bs[buf][brow + 32 * j];
      sb[j] = __builtin_amdgcn_perm(rb[1], rb[0], sel);
    }
    MxFrag8 f0, f1;
    mx_dma_frags8(f0, Acur, Bcur, 0, h, sw);
    mx_dma_substep8<0>(acc, f0, f1, Acur, Bcur, h, sw, sa, sb);
    mx_dma_substep8<1>(acc, f1, f0, Acur, Bcur, h, sw, sa, sb);
    mx_dma_substep8<2>(acc, f0, f1, Acur, Bcur, h, sw, sa, sb);
    mx_dma_substep8<3>(acc, f1, f0, Acur, Bcur, h, sw, sa, sb);
    mx_wait_vm0();
    __syncthreads();
  }
  // epilogue: rows wm * 128 + ..., columns wn * 64 + ...
  if (m0 + MTM <= M && n0 + MTN <= N && N <= (1 << 20)) {
    // Whole tile: a buffer resource from the tile's first element, 32-bit
    // offsets (256 rows of at most 2^20 floats stay below 2^30 bytes) and
    // uniform row offsets; each store writes two whole 128-byte lines of C,
    // which is written once: non-temporal.
    const int ld = (int)N;
    const __amdgpu_buffer_rsrc_t cr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(C + m0 * N + n0), 0, MTM * ld * 4, kBufferWord3);
    const int vo = ((wm * 128 + 4 * (lane >> 5)) * ld + wn * 64 + (lane & 31)) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int so = (i * 32 + 8 * (e >> 2) + (e & 3)) * ld * 4;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][e]), cr, vo + j * 128, so, kStreamLoad);
      }
    return;
  }
  float* Cw = C + (m0 + wm * 128 + 4 * (lane >> 5)) * N + n0 + wn * 64 + (lane & 31);
  const int64_t rlim = M - (m0 + wm * 128 + 4 * (lane >> 5)), clim = N - (n0 + wn * 64 + (lane & 31));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = i * 32 + 8 * (e >> 2) + (e & 3), cc = j * 32;
        if (r < rlim && cc < clim) Cw[r * N + cc] = acc[i][j][e];
      }
}

}  // namespace nvfp4

// ============================================================ host entry points
namespace {

using namespace nvfp4;

// One pass: every lane takes its kMxU quarter blocks once (the grid-stride
// loop only runs past 2^30 workgroups).  Workgroups are dispatched in order,
// so the stores in flight stay close together; 16 resident workgroups per CU
// striding over the whole tensor ran the 64 x 2048 x 7168 quantize in
// 0.51 ms against 0.395 ms, the dequantize in 0.505 against 0.42 ms.
int mx_grid(int64_t nq) {
  const int64_t most = std::max<int64_t>(1, (nq + (int64_t)kThreads * kMxU - 1) / ((int64_t)kThreads * kMxU));
  return (int)std::min<int64_t>(most, (int64_t)1 << 30);
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sf,
                                  void* stream) {
  if (rows < 0 || cols < 0 || cols % kMxBlock) return NVFP4_EINVAL;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (!x || !q || !sf) return NVFP4_EINVAL;
  if (rows > INT64_MAX / cols) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(x) || !nvfp4host::aligned16(q)) return NVFP4_EALIGN;
  nvfp4_status st = nvfp4host::check_device();
  if (st) return st;
  const int64_t nq = rows * cols / 8;
  mx_quantize_kernel<<<mx_grid(nq), kThreads, 0, (hipStream_t)stream>>>((const u32x4*)x, nq, (uint32_t*)q, sf);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

nvfp4_status nvfp4_mxfp4_dequantize(const uint8_t* q, const uint8_t* sf, int64_t rows, int64_t cols, uint16_t* y,
                                    void* stream) {
  if (rows < 0 || cols < 0 || cols % kMxBlock) return NVFP4_EINVAL;
  if (rows == 0 || cols == 0) return NVFP4_OK;
  if (!q || !sf || !y) return NVFP4_EINVAL;
  if (rows > INT64_MAX / cols) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(q) || !nvfp4host::aligned16(y)) return NVFP4_EALIGN;
  nvfp4_status st = nvfp4host::check_device();
  if (st) return st;
  const int64_t nq = rows * cols / 8;
  mx_dequant_kernel<<<mx_grid(nq), kThreads, 0, (hipStream_t)stream>>>((const uint32_t*)q, sf, nq, (u32x4*)y);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

nvfp4_status nvfp4_mxfp4_gemm(const uint8_t* a_q, const uint8_t* a_sf, const uint8_t* b_q, const uint8_t* b_sf,
                              int64_t M, int64_t N, int64_t K, float* c, void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % kMxBlock) return NVFP4_EINVAL;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!c) return NVFP4_EINVAL;
  if (K > 0 && (!a_q || !a_sf || !b_q || !b_sf)) return NVFP4_EINVAL;
  if ((M + MTM - 1) / MTM > 65535 || (N + MTN - 1) / MTN > 2147483647LL) return NVFP4_EINVAL;
  if (K > (1LL << 23)) return NVFP4_EINVAL;   // a workgroup's 256-row slab uses 32-bit offsets
  if (!nvfp4host::aligned16(a_q) || !nvfp4host::aligned16(b_q) || !nvfp4host::aligned16(c)) return NVFP4_EALIGN;
  nvfp4_status st = nvfp4host::check_device();
  if (st) return st;
  const dim3 grid((unsigned)((N + MTN - 1) / MTN), (unsigned)((M + MTM - 1) / MTM));
  // aligned path: whole K steps and 8-byte aligned scale rows
  const bool aligned = K % MTK == 0 && (reinterpret_cast<uintptr_t>(a_sf) & 7u) == 0 &&
                       (reinterpret_cast<uintptr_t>(b_sf) & 7u) == 0;
  if (aligned)
    mx_gemm_dma8_kernel<<<grid, MThreads8, 0, (hipStream_t)stream>>>(a_q, a_sf, b_q, b_sf, M, N, K, c);
  else
    mx_gemm_kernel<false><<<grid, MThreads, 0, (hipStream_t)stream>>>(a_q, a_sf, b_q, b_sf, M, N, K, c);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

}  // extern "C"
