// Quantize variants of the NVFP4 training recipe (axbrief.com, "NVFP4: how
// NVIDIA pre-trained a 12B model on 10 trillion tokens", section "Four
// stabilizers for training: from RHT to stochastic rounding"):
//   COLWISE  quantize x^T: blocks run down x's columns (the Dgrad / Wgrad
//            operand layout, contraction over x's rows)
//   2D       one E4M3 scale per 16 x 16 tile (weights), stored for each of
//            the tile's rows in the usual [rows][cols/16] layout, so a
//            weight and its transpose quantize to the same values
//   RHT      each 16-value block becomes H16 (s .* x) / 4 before quantizing
//            (H16 the Sylvester Hadamard matrix, s the caller's +-1 signs),
//            computed in fp32 as the fast Walsh-Hadamard transform, stages
//            h = 1, 2, 4, 8, then * 1/4
//   SR       the element rounding onto E2M1 is stochastic: with lo <= y < hi
//            neighbouring E2M1 magnitudes, round up when u16 / 2^16 <
//            (y - lo) / (hi - lo); u16 is 16 bits of Philox4x32-10 (Salmon
//            et al., SC 2011) keyed by the seed, counter (n, n >> 32, 0, 0)
//            with n = i / 8 + offset for output element i, half (i mod 2) of
//            word (i mod 8) / 2.  Scales stay round-to-nearest.
// Everything else is the two-level recipe (tensor amax -> g, block amax ->
// E4M3 scale, element quotients), applied to the (transformed) fp32 values.
// The quotients use the fp64-reciprocal method of the codec: its exactness
// argument holds for any fp32 numerator (see common.hpp).
//
// Work unit: one wave takes a 16-row x 64-column group of x; lane L holds
// row L % 16 of the 16 x 16 tile L / 16 (16 values, one block).  COLWISE
// transposes the group through LDS so that lane L then holds column
// 16 (L / 16) + L % 16 of the group.  Two passes, each reading x once: the
// amax pass (transformed values, per-workgroup partial maxima) and the
// encode pass.
#include <algorithm>

#include "common.hpp"

namespace nvfp4 {

constexpr int kVarThreads = 256;
constexpr int kVarMaxPartials = 2048;
constexpr int kGroupRows = 16, kGroupCols = 64;
constexpr int kTRow = kGroupCols + 8;          // LDS row of a transpose buffer (bf16 units, 16-byte rows)

struct VarShape {
  int64_t rows, cols, n;                       // per tensor
  int64_t grp_r, grp_c;                        // groups down and across
  int64_t R, C;                                // output matrix per tensor
};

// The lane's 16 values of group gidx (rows 16 gr.., columns 64 gc + 16 t4..)
// as fp32, transposed for COLWISE, with the output row it belongs to and
// its block index in that row; valid is false for lanes past the tensor.
template <bool kColwise>
__device__ __forceinline__ bool load_block(const uint16_t* __restrict__ xt, const VarShape& sh, int64_t gidx,
                                           uint16_t (*tb)[kTRow], float (&v)[16], int64_t& orow, int64_t& oblk) {
  const int lane = threadIdx.x & 63, r = lane & 15, t4 = lane >> 4;
  const int64_t gr = gidx / sh.grp_c, gc = gidx % sh.grp_c;
  const int64_t row = gr * kGroupRows + r, col0 = gc * kGroupCols + 16 * t4;
  const bool in = row < sh.rows && col0 < sh.cols;
  u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
  if (in) {
    const u32x4* p = (const u32x4*)(xt + row * sh.cols + col0);
    a = p[0];
    b = p[1];
  }
  if (!kColwise) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_lo(w[i]);
      v[2 * i + 1] = bf16_hi(w[i]);
    }
    orow = row;
    oblk = col0 / 16;
    return in;
  }
  // transpose through this wave's LDS buffer: tb[r][16 t4 + j] = x[row][col0 + j]
  *(u32x4*)&tb[r][16 * t4] = a;
  *(u32x4*)&tb[r][16 * t4 + 8] = b;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int c = 16 * t4 + r;                    // the group column this lane now holds
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = __uint_as_float((uint32_t)tb[j][c] << 16);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();              // reads done before the next group's writes
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  orow = gc * kGroupCols + c;
  oblk = gr;
  return orow < sh.cols;
}

// v <- H16 (s .* v) / 4, fast Walsh-Hadamard stages h = 1, 2, 4, 8 (fp32).
__device__ __forceinline__ void rht16(float (&v)[16], uint32_t signs) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if ((signs >> j) & 1u) v[j] = -v[j];
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = v[j] * 0.25f;
}

__device__ __forceinline__ uint32_t absmax_bits(const float (&v)[16]) {
  uint32_t m = 0u;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t b = __float_as_uint(v[j]) & 0x7fffffffu;   // order-preserving for |v|
    m = m > b ? m : b;
  }
  return m;
}

// Philox4x32-10 (Salmon et al., SC 2011).
__device__ __forceinline__ void philox(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1, uint32_t (&o)[4]) {
  uint32_t c2 = 0u, c3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
    const uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  o[0] = c0;
  o[1] = c1;
  o[2] = c2;
  o[3] = c3;
}

// Stochastic E2M1 magnitude code of y >= 0 with the 16-bit draw u.
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u) {
  if (y >= 6.0f) return 7u;
  const uint32_t k = (uint32_t)(y >= 0.5f) + (uint32_t)(y >= 1.0f) + (uint32_t)(y >= 1.5f) + (uint32_t)(y >= 2.0f) +
                     (uint32_t)(y >= 3.0f) + (uint32_t)(y >= 4.0f);
  // lower neighbour and 1 / gap (gaps are powers of two, so p is exact)
  const float lo = k <= 4u ? 0.5f * (float)k : k == 5u ? 3.0f : 4.0f;
  const float inv_gap = k < 4u ? 2.0f : k < 6u ? 1.0f : 0.5f;
  const float p = (y - lo) * inv_gap;
  return k + ((float)u < p * 65536.0f ? 1u : 0u);
}

template <bool kColwise, bool kRht>
__global__ void __launch_bounds__(kVarThreads) var_amax_kernel(const uint16_t* __restrict__ x, VarShape sh,
                                                               uint32_t signs, uint32_t* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t tbuf[kVarThreads / 64][kGroupRows][kTRow];
  __shared__ uint32_t red[kVarThreads / 64];
  const int t = blockIdx.y, wave = wave_id();
  const uint16_t* xt = x + (int64_t)t * sh.n;
  const int64_t ngroups = sh.grp_r * sh.grp_c;
  uint32_t m = 0u;
  for (int64_t gidx = (int64_t)blockIdx.x * (kVarThreads / 64) + wave; gidx < ngroups;
       gidx += (int64_t)gridDim.x * (kVarThreads / 64)) {
    float v[16];
    int64_t orow, oblk;
    const bool in = load_block<kColwise>(xt, sh, gidx, tbuf[wave], v, orow, oblk);
    if (kRht) rht16(v, signs);
    const uint32_t b = absmax_bits(v);
    if (in) m = m > b ? m : b;                   // invalid lanes hold zeros anyway
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kVarThreads / 64; ++w) r = r > red[w] ? r : red[w];
    partial[(int64_t)t * gridDim.x + blockIdx.x] = r;
  }
}

template <bool kColwise, bool k2D, bool kRht, bool kSr>
__global__ void __launch_bounds__(kVarThreads) var_encode_kernel(const uint16_t* __restrict__ x, VarShape sh,
                                                                 uint32_t signs, uint64_t seed, uint64_t offset,
                                                                 const uint32_t* __restrict__ partial, int npartial,
                                                                 uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
                                                                 float* __restrict__ gout) {
  __shared__ __attribute__((aligned(16))) uint16_t tbuf[kVarThreads / 64][kGroupRows][kTRow];
  __shared__ double table[128];
  __shared__ uint32_t red[kVarThreads / 64];
  const int t = blockIdx.y, wave = wave_id(), lane = threadIdx.x & 63;
  // g = RN32(amax / 2688) from the amax pass's partials (fp32 bits)
  uint32_t am = 0u;
  for (int i = threadIdx.x; i < npartial; i += kVarThreads) {
    const uint32_t p = partial[(int64_t)t * npartial + i];
    am = am > p ? am : p;
  }
  am = wave_max_u32(am);
  if (lane == 0) red[wave] = am;
  __syncthreads();
  am = red[0];
#pragma unroll
  for (int w = 1; w < kVarThreads / 64; ++w) am = am > red[w] ? am : red[w];
  const float g = __uint_as_float(am) / kGlobalDiv;
  if (blockIdx.x == 0 && threadIdx.x == 0) gout[t] = g;
  for (uint32_t j = threadIdx.x; j < 127u; j += kVarThreads) table[j] = recip_entry(j, g);
  const double r6 = recip_d6(g);
  __syncthreads();

  const uint16_t* xt = x + (int64_t)t * sh.n;
  const int64_t ngroups = sh.grp_r * sh.grp_c;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int64_t gidx = (int64_t)blockIdx.x * (kVarThreads / 64) + wave; gidx < ngroups;
       gidx += (int64_t)gridDim.x * (kVarThreads / 64)) {
    float v[16];
    int64_t orow, oblk;
    const bool in = load_block<kColwise>(xt, sh, gidx, tbuf[wave], v, orow, oblk);
    if (kRht) rht16(v, signs);
    uint32_t bam = absmax_bits(v);
    if (k2D) {                                   // the tile's 16 lanes: same lane / 16
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)bam, off, 64);
        bam = bam > o ? bam : o;
      }
    }
    const uint32_t sbyte = e4m3_rne_sat(rn32((double)__uint_as_float(bam) * r6));
    const double rd = table[sbyte];
    uint32_t code[16];
    if (kSr) {
      // output element index of this block's first value; 16 values use two counters
      const int64_t i0 = ((int64_t)t * sh.R + orow) * sh.C + 16 * oblk;
      const uint64_t n = (uint64_t)i0 / 8 + offset;
      uint32_t w0[4], w1[4];
      philox((uint32_t)n, (uint32_t)(n >> 32), k0, k1, w0);
      philox((uint32_t)(n + 1), (uint32_t)((n + 1) >> 32), k0, k1, w1);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t word = j < 8 ? w0[(j & 7) >> 1] : w1[(j & 7) >> 1];
        const uint32_t u = (word >> (16 * (j & 1))) & 0xffffu;
        const float y = rn32((double)fabsf(v[j]) * rd);
        code[j] = (__float_as_uint(v[j]) >> 31 << 3) | e2m1_sr(y, u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const uint32_t pr = fp4_pair<0>(0u, rn32((double)v[j] * rd), rn32((double)v[j + 1] * rd));
        code[j] = pr & 15u;
        code[j + 1] = (pr >> 4) & 15u;
      }
    }
    if (in) {
      u32x2 packed = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) packed[j / 4] |= (code[2 * j] | (code[2 * j + 1] << 4)) << (8 * (j % 4));
      *(u32x2*)(q + (((int64_t)t * sh.R + orow) * sh.C + 16 * oblk) / 2) = packed;
      sf[((int64_t)t * sh.R + orow) * (sh.C / 16) + oblk] = (uint8_t)sbyte;
    }
  }
}

}  // namespace nvfp4

// ============================================================ host entry point
namespace {

using namespace nvfp4;

int var_wgs(int64_t batch, int64_t ngroups) {
  const int64_t target = std::max<int64_t>(1, (int64_t)nvfp4host::num_cus() * 8 / std::max<int64_t>(1, batch));
  const int64_t need = (ngroups + kVarThreads / 64 - 1) / (kVarThreads / 64);
  return (int)std::max<int64_t>(1, std::min<int64_t>(std::min(target, need), kVarMaxPartials));
}

template <bool kColwise, bool k2D, bool kRht, bool kSr>
void launch_encode(dim3 grid, hipStream_t s, const uint16_t* x, const VarShape& sh, uint32_t signs, uint64_t seed,
                   uint64_t offset, const uint32_t* partial, uint8_t* q, uint8_t* sf, float* g) {
  var_encode_kernel<kColwise, k2D, kRht, kSr><<<grid, kVarThreads, 0, s>>>(x, sh, signs, seed, offset, partial,
                                                                           (int)grid.x, q, sf, g);
}

}  // namespace

extern "C" {

size_t nvfp4_quantize_ex_workspace_bytes(int64_t batch) {
  return batch <= 0 ? 0 : (size_t)batch * kVarMaxPartials * sizeof(uint32_t);
}

nvfp4_status nvfp4_quantize_ex(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint32_t variant,
                               uint32_t rht_signs, uint64_t seed, uint64_t offset, uint8_t* q, uint8_t* sf, float* g,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || rows < 0 || cols < 0 || cols % kBlock) return NVFP4_EINVAL;
  if (variant & ~(uint32_t)(NVFP4_VAR_COLWISE | NVFP4_VAR_2D | NVFP4_VAR_RHT | NVFP4_VAR_SR)) return NVFP4_EINVAL;
  if (rht_signs > 0xffffu) return NVFP4_EINVAL;
  const bool colwise = variant & NVFP4_VAR_COLWISE, two_d = variant & NVFP4_VAR_2D;
  const bool rht = variant & NVFP4_VAR_RHT;
  if ((colwise || two_d) && rows % 16) return NVFP4_EINVAL;
  if (two_d && rht) return NVFP4_ENOTSUP;
  if (batch == 0) return NVFP4_OK;
  if (!g) return NVFP4_EINVAL;
  if (batch > 65535) return NVFP4_EINVAL;
  if (rows > 0 && cols > INT64_MAX / rows / batch) return NVFP4_EINVAL;
  const int64_t n = rows * cols;
  if (n > 0 && (!x || !q || !sf)) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(x) || !nvfp4host::aligned16(q)) return NVFP4_EALIGN;
  if (reinterpret_cast<uintptr_t>(g) & 3u) return NVFP4_EALIGN;
  if (!workspace || workspace_bytes < nvfp4_quantize_ex_workspace_bytes(batch)) return NVFP4_EWORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 3u) return NVFP4_EALIGN;
  nvfp4_status st = nvfp4host::check_device();
  if (st) return st;
  VarShape sh;
  sh.rows = rows;
  sh.cols = cols;
  sh.n = n;
  sh.grp_r = (rows + kGroupRows - 1) / kGroupRows;
  sh.grp_c = (cols + kGroupCols - 1) / kGroupCols;
  sh.R = colwise ? cols : rows;
  sh.C = colwise ? rows : cols;
  const int64_t ngroups = sh.grp_r * sh.grp_c;
  const dim3 grid((unsigned)var_wgs(batch, ngroups), (unsigned)batch);
  hipStream_t s = (hipStream_t)stream;
  uint32_t* partial = (uint32_t*)workspace;
  // pass 1: the amax of the quantized values (the orientation matters only under RHT)
  if (rht && colwise)
    var_amax_kernel<true, true><<<grid, kVarThreads, 0, s>>>(x, sh, rht_signs, partial);
  else if (rht)
    var_amax_kernel<false, true><<<grid, kVarThreads, 0, s>>>(x, sh, rht_signs, partial);
  else
    var_amax_kernel<false, false><<<grid, kVarThreads, 0, s>>>(x, sh, rht_signs, partial);
  NVFP4_LAUNCH_CHECK();
  // pass 2: scales and codes
  switch (variant) {
#define NVFP4_VAR_CASE(V)                                                                                  \
  case V:                                                                                                  \
    launch_encode<(V & NVFP4_VAR_COLWISE) != 0, (V & NVFP4_VAR_2D) != 0, (V & NVFP4_VAR_RHT) != 0,         \
                  (V & NVFP4_VAR_SR) != 0>(grid, s, x, sh, rht_signs, seed, offset, partial, q, sf, g);     \
    break;
    NVFP4_VAR_CASE(0) NVFP4_VAR_CASE(1) NVFP4_VAR_CASE(2) NVFP4_VAR_CASE(3)
    NVFP4_VAR_CASE(4) NVFP4_VAR_CASE(5) NVFP4_VAR_CASE(8) NVFP4_VAR_CASE(9)
    NVFP4_VAR_CASE(10) NVFP4_VAR_CASE(11) NVFP4_VAR_CASE(12) NVFP4_VAR_CASE(13)
#undef NVFP4_VAR_CASE
    default: return NVFP4_ENOTSUP;               // 2D with RHT (rejected above)
  }
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

}  // extern "C"
