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
// Work unit: a strip of 16 rows x 512 columns per wave.  Lane l holds
// columns 8l..8l+7 of each of the 16 rows (16 loads of 16 bytes, each
// instruction one contiguous kilobyte).  Row-wise, a block is the lane pair
// (2m, 2m+1) within a row; COLWISE, a block is one column of the strip, all
// in one lane, so x^T needs no data exchange.  2D tiles are the lane pair
// over all 16 rows.  RHT runs in registers (across the pair for its last
// stage row-wise).  A wave walks a run of strips down one 512-column band,
// so COLWISE writes whole stretches of each output row in turn.  Two
// passes, each reading x once: the amax of the quantized values, then the
// encode.
#include <algorithm>

#include "common.hpp"

namespace nvfp4 {

constexpr int kVarThreads = 256;
constexpr int kVarMaxPartials = 2048;
constexpr int kStripRows = 16, kStripCols = 512;

struct VarShape {
  int64_t rows, cols, n;                       // per tensor
  int64_t R, C;                                // output matrix per tensor
  int64_t sr, sc;                              // strips down and across
  int64_t seg, nseg, nitems;                   // strips per work item, items per band, items per tensor
};

// Philox4x32-10 (Salmon et al., SC 2011).  The ten round keys are computed
// once per thread and held in VGPRs: uniform as they are, as scalars they
// would not fit beside the kernels' other uniform values and were spilled
// to VGPR lanes and read back (v_readlane) inside the loops.
struct PhiloxKeys {
  uint32_t k0[10], k1[10];
};

__device__ __forceinline__ PhiloxKeys philox_keys(uint64_t seed) {
  PhiloxKeys k;
  uint32_t a = (uint32_t)seed, b = (uint32_t)(seed >> 32);
  asm volatile("v_mov_b32 %0, %1" : "=v"(a) : "s"(a));   // keep the keys in vector registers
  asm volatile("v_mov_b32 %0, %1" : "=v"(b) : "s"(b));
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    k.k0[r] = a;
    k.k1[r] = b;
    a += 0x9E3779B9u;
    b += 0xBB67AE85u;
  }
  return k;
}

__device__ __forceinline__ void philox(uint32_t c0, uint32_t c1, const PhiloxKeys& k, uint32_t (&o)[4]) {
  uint32_t c2 = 0u, c3 = 0u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // one 32 x 32 -> 64-bit multiply each (a single v_mad_u64_u32)
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u, p1 = (uint64_t)c2 * 0xCD9E8D57u;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    // the three-way xors as single v_bitop3 (0x96 is a ^ b ^ c)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k.k0[r], 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k.k1[r], 0x96);
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

// The 8 16-bit draws of output elements 8n'..8n'+7, n' = n - offset.
__device__ __forceinline__ void draws8(uint64_t n, const PhiloxKeys& k, uint32_t (&u)[8]) {
  uint32_t w[4];
  philox((uint32_t)n, (uint32_t)(n >> 32), k, w);
#pragma unroll
  for (int j = 0; j < 8; ++j) u[j] = (w[j >> 1] >> (16 * (j & 1))) & 0xffffu;
}

// Stochastic E2M1 magnitude code of y >= 0 with the 16-bit draw u: the grid
// point below y, plus one when u / 2^16 < (y - lo) / gap.
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t u) {
  const uint32_t b = __float_as_uint(y);
  // y >= 1: the gap is half the binade and the fraction is the low 22
  // mantissa bits m, so the rule reads m > 64 u.  Adding 2^22 - 1 - 64 u
  // carries into bit 22 exactly then; bits 22 and up then read 254 + code
  // (1.0 is 254, 6.0 is 259, larger y saturate to code 7).  The xor forms
  // 2^22 - 1 - 64 u and subtracts 252 << 22 in one constant.
  uint32_t cn = (((u << 6) ^ 0xC13FFFFFu) + b) >> 22;
  cn = cn < 7u ? cn : 7u;
  // y < 1: the grid is 0, 0.5, 1 with gap 0.5.  With F = 2^17 y (exact) and
  // k = floor(F / 2^16) the lower point, the rule reads u < F - 2^16 k; u is
  // an integer, so that is u + 2^16 k <= ceil(F) - 1, and the code is
  // (ceil(F) + 2^16 - 1 - u) >> 16 (u ^ 0xFFFF = 2^16 - 1 - u).
  const uint32_t cf = ((u ^ 0xFFFFu) + (uint32_t)__builtin_ceilf(y * 131072.0f)) >> 16;
  return b >= 0x3F800000u ? cn : cf;
}

// fp32 value of element j (0..7) of a row chunk of 8 bf16.
__device__ __forceinline__ float chunk_val(const u32x4& c, int j) {
  const uint32_t w = j < 2 ? c.x : j < 4 ? c.y : j < 6 ? c.z : c.w;
  return (j & 1) ? bf16_hi(w) : bf16_lo(w);
}

__device__ __forceinline__ float dpp_swap_pair(float v) {     // lane ^ 1
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t pair_max_u32(uint32_t m) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false);
  return m > o ? m : o;
}
__device__ __forceinline__ uint32_t fabs_bits(float v) { return __float_as_uint(v) & 0x7fffffffu; }

// v <- H16 (s .* v) / 4 for a block held in one lane (fp32, stages 1, 2, 4, 8).
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

// The same for a block split over a lane pair: this lane holds elements
// 8 (lane & 1) .. +7; stages 1, 2, 4 in registers, stage 8 across the pair.
__device__ __forceinline__ void rht16_pair(float (&v)[8], uint32_t signs, bool odd) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if ((signs >> (j + (odd ? 8 : 0))) & 1u) v[j] = -v[j];
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float o = dpp_swap_pair(v[j]);          // even lane: a = own, b = o; odd lane: a = o, b = own
    v[j] = (odd ? o - v[j] : v[j] + o) * 0.25f;
  }
}

// Keeps a per-row pointer or counter a value that steps by one add per row:
// without it the compiler precomputes all 16 rows' offsets as scalars
// outside the loops, which spills scalar registers to vector lanes.
template <typename T>
__device__ __forceinline__ void step_opaque(T& v) {
  asm volatile("" : "+v"(v));
}

// Loads strip (sr_i, band) of tensor t: raw[r] = row r0 + r, columns
// 512 band + 8 lane .. +7 (zeros past the tensor).
__device__ __forceinline__ void load_strip(const uint16_t* __restrict__ xt, const VarShape& sh, int64_t r0,
                                           int64_t col, u32x4 (&raw)[kStripRows]) {
  const bool cin = col < sh.cols;
  const uint16_t* p = xt + r0 * sh.cols + col;
#pragma unroll
  for (int r = 0; r < kStripRows; ++r) {
    raw[r] = u32x4{0u, 0u, 0u, 0u};
    if (cin && r0 + r < sh.rows) raw[r] = __builtin_nontemporal_load((const u32x4*)p);
    p += sh.cols;
    step_opaque(p);
  }
}

// Work item it -> band (512-column band) and its strips [s0, s1).
__device__ __forceinline__ void var_item(const VarShape& sh, int64_t it, int64_t& band, int64_t& s0, int64_t& s1) {
  band = it / sh.nseg;
  s0 = (it % sh.nseg) * sh.seg;
  s1 = s0 + sh.seg < sh.sr ? s0 + sh.seg : sh.sr;
}

template <bool kColwise, bool kRht>
__global__ void __launch_bounds__(kVarThreads) var_amax_kernel(const uint16_t* __restrict__ x, VarShape sh,
                                                               uint32_t signs, uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kVarThreads / 64];
  const int t = blockIdx.y, wave = wave_id(), lane = threadIdx.x & 63;
  const uint16_t* xt = x + (int64_t)t * sh.n;
  uint32_t m = 0u;
  for (int64_t it = (int64_t)blockIdx.x * (kVarThreads / 64) + wave; it < sh.nitems;
       it += (int64_t)gridDim.x * (kVarThreads / 64)) {
    int64_t band, s0, s1;
    var_item(sh, it, band, s0, s1);
    const int64_t col = band * kStripCols + 8 * lane;
    for (int64_t si = s0; si < s1; ++si) {
      u32x4 raw[kStripRows];
      load_strip(xt, sh, si * kStripRows, col, raw);
      if (!kRht) {                                     // the amax of x itself
        uint32_t pk = 0u;
#pragma unroll
        for (int r = 0; r < kStripRows; ++r)
          pk = pk_absmax(pk_absmax(pk_absmax(pk_absmax(pk, raw[r].x), raw[r].y), raw[r].z), raw[r].w);
        const uint32_t b = halves_max(pk) << 16;       // bf16 magnitude -> fp32 bits
        m = m > b ? m : b;
      } else if (kColwise) {                           // blocks down the lane's 8 columns
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = chunk_val(raw[r], j);
          rht16(v, signs);
#pragma unroll
          for (int r = 0; r < 16; ++r) m = m > fabs_bits(v[r]) ? m : fabs_bits(v[r]);
        }
      } else {                                         // blocks across the lane pair of each row
#pragma unroll
        for (int r = 0; r < kStripRows; ++r) {
          float v[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = chunk_val(raw[r], j);
          rht16_pair(v, signs, lane & 1);
#pragma unroll
          for (int j = 0; j < 8; ++j) m = m > fabs_bits(v[j]) ? m : fabs_bits(v[j]);
        }
      }
    }
  }
  m = wave_max_u32(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = red[0];
#pragma unroll
    for (int w = 1; w < kVarThreads / 64; ++w) r = r > red[w] ? r : red[w];
    partial[(int64_t)t * gridDim.x + blockIdx.x] = r;
  }
}

// Codes of n values (n = 8 or 16) with reciprocal rd, RNE or stochastic
// with draws u; packed 2 per byte (element 2i in the low nibble).
template <int kN, bool kSr>
__device__ __forceinline__ void encode_vals(const float (&v)[kN], double rd, const uint32_t (&u)[kN],
                                            uint32_t (&out)[kN / 8]) {
#pragma unroll
  for (int w = 0; w < kN / 8; ++w) out[w] = 0u;
  if (kSr) {
#pragma unroll
    for (int j = 0; j < kN; ++j) {
      const float y = rn32((double)fabsf(v[j]) * rd);
      const uint32_t c = (__float_as_uint(v[j]) >> 31 << 3) | e2m1_sr(y, u[j]);
      out[j / 8] |= c << (4 * (j % 8));
    }
  } else {
#pragma unroll
    for (int j = 0; j < kN; j += 8) {
      uint32_t c = fp4_pair<0>(0u, rn32((double)v[j] * rd), rn32((double)v[j + 1] * rd));
      c = fp4_pair<1>(c, rn32((double)v[j + 2] * rd), rn32((double)v[j + 3] * rd));
      c = fp4_pair<2>(c, rn32((double)v[j + 4] * rd), rn32((double)v[j + 5] * rd));
      out[j / 8] = fp4_pair<3>(c, rn32((double)v[j + 6] * rd), rn32((double)v[j + 7] * rd));
    }
  }
}

// Row-wise encode (the COLWISE layout has its own kernel below).
template <bool k2D, bool kRht, bool kSr>
__global__ void __launch_bounds__(kVarThreads) var_encode_kernel(const uint16_t* __restrict__ x, VarShape sh,
                                                                 uint32_t signs, uint64_t seed, uint64_t offset,
                                                                 const uint32_t* __restrict__ partial, int npartial,
                                                                 uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
                                                                 float* __restrict__ gout) {
  __shared__ double table[128];
  __shared__ uint32_t red[kVarThreads / 64];
  const int t = blockIdx.y, wave = wave_id(), lane = threadIdx.x & 63;
  const bool odd = lane & 1;
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
  const PhiloxKeys pk = philox_keys(seed);
  // per output row: C / 2 code bytes, C / 16 scale bytes, C / 8 draw counters
  const int64_t qstep = sh.C / 2, sstep = sh.C / 16, nstep = sh.C / 8;
  for (int64_t it = (int64_t)blockIdx.x * (kVarThreads / 64) + wave; it < sh.nitems;
       it += (int64_t)gridDim.x * (kVarThreads / 64)) {
    int64_t band, s0, s1;
    var_item(sh, it, band, s0, s1);
    const int64_t col = band * kStripCols + 8 * lane;
    const bool cin = col < sh.cols;
    for (int64_t si = s0; si < s1; ++si) {
      const int64_t r0 = si * kStripRows;
      u32x4 raw[kStripRows];
      load_strip(xt, sh, r0, col, raw);
      uint32_t tile = 0u;                              // 2D: the tile amax (fp32 bits), pair-wide
      if (k2D) {
        uint32_t pm = 0u;
#pragma unroll
        for (int r = 0; r < kStripRows; ++r)
          pm = pk_absmax(pk_absmax(pk_absmax(pk_absmax(pm, raw[r].x), raw[r].y), raw[r].z), raw[r].w);
        tile = pair_max_u32(halves_max(pm) << 16);
      }
      // row r0's codes, scale byte and first draw counter; the rows below
      // step by one output row each
      const int64_t orow0 = (int64_t)t * sh.R + r0;
      uint8_t* qr = q + orow0 * qstep + col / 2;
      uint8_t* sr = sf + orow0 * sstep + col / 16;
      uint64_t n = (uint64_t)(orow0 * nstep + col / 8) + offset;
      const int nrows = (int)(sh.rows - r0 < kStripRows ? sh.rows - r0 : kStripRows);
      // row r: this lane's half of block (col / 16), the partner holds the other half
#pragma unroll
      for (int r = 0; r < kStripRows; ++r) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = chunk_val(raw[r], j);
        if (kRht) rht16_pair(v, signs, odd);
        uint32_t bam;
        if (k2D) {
          bam = tile;
        } else {
          bam = 0u;
#pragma unroll
          for (int j = 0; j < 8; ++j) bam = bam > fabs_bits(v[j]) ? bam : fabs_bits(v[j]);
          bam = pair_max_u32(bam);
        }
        const uint32_t sbyte = e4m3_rne_sat(rn32((double)__uint_as_float(bam) * r6));
        uint32_t u[8];
        if (kSr) draws8(n, pk, u);
        uint32_t codes[1];
        encode_vals<8, kSr>(v, table[sbyte], u, codes);
        if (cin && r < nrows) {
          *(uint32_t*)qr = codes[0];
          if (!odd) *sr = (uint8_t)sbyte;
        }
        qr += qstep;
        sr += sstep;
        n += nstep;
        step_opaque(qr);
        step_opaque(sr);
        step_opaque(n);
      }
    }
  }
}

// COLWISE encode, one workgroup per block of 16 strips (256 rows) of a
// 512-column band: the four waves encode 4 strips each into LDS, then the
// workgroup writes each output row's 128 code bytes (and 16 scale bytes) of
// the block as whole cache lines.
//   codes: output row r, strip k at 8-byte slot k ^ 2 ((r >> 3) & 7) of the
//          row's 128 bytes (the XOR spreads a wave's writes, 8 rows per lane,
//          over the banks; slot pairs 2p, 2p + 1 stay together and in order)
//   scales: strip-major, 512 bytes per strip
constexpr int kColStrips = 16;

struct VarColSmem {
  uint32_t codes[kStripCols][kColStrips * 2];
  uint8_t scales[kColStrips][kStripCols];
};

__device__ __forceinline__ int col_slot(int r, int k) { return k ^ (2 * ((r >> 3) & 7)); }

template <bool k2D, bool kRht, bool kSr>
__global__ void __launch_bounds__(kVarThreads) var_encode_colwise_kernel(
    const uint16_t* __restrict__ x, VarShape sh, uint32_t signs, uint64_t seed, uint64_t offset,
    const uint32_t* __restrict__ partial, int npartial, uint8_t* __restrict__ q, uint8_t* __restrict__ sf,
    float* __restrict__ gout) {
  __shared__ double table[128];
  __shared__ uint32_t red[kVarThreads / 64];
  __shared__ __attribute__((aligned(16))) VarColSmem cs;
  const int t = blockIdx.y, wave = wave_id(), lane = threadIdx.x & 63;
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
  const PhiloxKeys pk = philox_keys(seed);
  const int64_t nblk = (sh.sr + kColStrips - 1) / kColStrips;
  const int64_t nitems = sh.sc * nblk;
  for (int64_t it = blockIdx.x; it < nitems; it += gridDim.x) {           // workgroup-uniform
    const int64_t band = it / nblk, blk = it % nblk;
    const int nstr = (int)std::min<int64_t>(kColStrips, sh.sr - blk * kColStrips);
    const int64_t col = band * kStripCols + 8 * lane;
    for (int k = wave; k < nstr; k += kVarThreads / 64) {
      const int64_t r0 = (blk * kColStrips + k) * kStripRows;
      u32x4 raw[kStripRows];
      load_strip(xt, sh, r0, col, raw);
      uint32_t tile = 0u;
      if (k2D) {
        uint32_t pk = 0u;
#pragma unroll
        for (int r = 0; r < kStripRows; ++r)
          pk = pk_absmax(pk_absmax(pk_absmax(pk_absmax(pk, raw[r].x), raw[r].y), raw[r].z), raw[r].w);
        tile = pair_max_u32(halves_max(pk) << 16);
      }
      uint32_t sb[2] = {0u, 0u};                   // columns j's scale bytes
      // draw counter of column col's block r0 / 16; each column is one output row on
      uint64_t n = (uint64_t)(((int64_t)t * sh.R + col) * (sh.C / 8) + r0 / 8) + offset;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = chunk_val(raw[r], j);
        if (kRht) rht16(v, signs);
        uint32_t bam = 0u;
        if (k2D) {
          bam = tile;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) bam = bam > fabs_bits(v[r]) ? bam : fabs_bits(v[r]);
        }
        const uint32_t sbyte = e4m3_rne_sat(rn32((double)__uint_as_float(bam) * r6));
        uint32_t u[16];
        if (kSr) {
          uint32_t u0[8], u1[8];
          draws8(n, pk, u0);
          draws8(n + 1, pk, u1);
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            u[kk] = u0[kk];
            u[kk + 8] = u1[kk];
          }
        }
        uint32_t codes[2];
        encode_vals<16, kSr>(v, table[sbyte], u, codes);
        const int r = 8 * lane + j;                // output row within the band
        *(u32x2*)&cs.codes[r][2 * col_slot(r, k)] = u32x2{codes[0], codes[1]};
        sb[j / 4] |= sbyte << (8 * (j % 4));
        n += (uint64_t)(sh.C / 8);
        step_opaque(n);
      }
      *(u32x2*)&cs.scales[k][8 * lane] = u32x2{sb[0], sb[1]};
    }
    __syncthreads();
    // each output row of the band gets nstr * 8 code bytes and nstr scale bytes
    const int rows_here = (int)std::min<int64_t>(kStripCols, sh.cols - band * kStripCols);
    const int64_t orow0 = (int64_t)t * sh.R + band * kStripCols;
    const bool q16 = sh.C % 32 == 0;               // output rows of codes start 16-byte aligned
#pragma unroll 4
    for (int i = 0; i < kStripCols * 8 / kVarThreads; ++i) {
      const int flat = i * kVarThreads + threadIdx.x;
      const int r = flat >> 3, pc = flat & 7;      // output row, 16-byte piece (strips 2 pc, 2 pc + 1)
      if (r < rows_here && 2 * pc < nstr) {
        const u32x4 v = *(const u32x4*)&cs.codes[r][2 * col_slot(r, 2 * pc)];
        uint8_t* dst = q + (orow0 + r) * (sh.C / 2) + blk * (kColStrips * 8) + 16 * pc;
        if (2 * pc + 1 < nstr && q16) {
          *(u32x4*)dst = v;
        } else {
          *(u32x2*)dst = u32x2{v.x, v.y};
          if (2 * pc + 1 < nstr) *(u32x2*)(dst + 8) = u32x2{v.z, v.w};
        }
      }
    }
    for (int r = threadIdx.x; r < rows_here; r += kVarThreads) {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < kColStrips; ++k) w[k / 4] |= (uint32_t)cs.scales[k][r] << (8 * (k % 4));
      uint8_t* dst = sf + (orow0 + r) * (sh.C / 16) + blk * kColStrips;
      if (nstr == kColStrips && !(reinterpret_cast<uintptr_t>(dst) & 15u)) {
        *(u32x4*)dst = u32x4{w[0], w[1], w[2], w[3]};
      } else {
        for (int k = 0; k < nstr; ++k) dst[k] = (uint8_t)(w[k / 4] >> (8 * (k % 4)));
      }
    }
    __syncthreads();                               // LDS free for the next block
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
  if (kColwise)
    var_encode_colwise_kernel<k2D, kRht, kSr><<<grid, kVarThreads, 0, s>>>(x, sh, signs, seed, offset, partial,
                                                                           (int)grid.x, q, sf, g);
  else
    var_encode_kernel<k2D, kRht, kSr><<<grid, kVarThreads, 0, s>>>(x, sh, signs, seed, offset, partial,
                                                                   (int)grid.x, q, sf, g);
}

}  // namespace

namespace nvfp4host {
// The single-launch 2D quantize (codec.hip): one read of the input when a
// tensor fits on chip; ENOTSUP otherwise.
size_t quantize_2d_onchip_ws_bytes(int64_t batch);
nvfp4_status quantize_2d_onchip(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, bool colwise, uint8_t* q,
                                uint8_t* sf, float* g, void* ws, hipStream_t s);
}  // namespace nvfp4host

extern "C" {

// Scratch: the single-launch 2D path's exchange header, then the two-pass
// path's per-workgroup partial maxima.
size_t nvfp4_quantize_ex_workspace_bytes(int64_t batch) {
  return batch <= 0 ? 0
                    : nvfp4host::quantize_2d_onchip_ws_bytes(batch) + (size_t)batch * kVarMaxPartials * sizeof(uint32_t);
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
  sh.R = colwise ? cols : rows;
  sh.C = colwise ? rows : cols;
  sh.sr = (rows + kStripRows - 1) / kStripRows;
  sh.sc = (cols + kStripCols - 1) / kStripCols;
  // strips per work item: enough items for about 16 waves per CU, at most 16 strips
  const int64_t strips = sh.sr * sh.sc * batch;
  sh.seg = std::max<int64_t>(1, std::min<int64_t>(16, strips / ((int64_t)nvfp4host::num_cus() * 16)));
  sh.nseg = (sh.sr + sh.seg - 1) / sh.seg;
  sh.nitems = sh.sc * sh.nseg;
  // workgroups: per-wave strip runs (row-wise), or per-workgroup blocks of 16 strips (COLWISE)
  const int64_t wgs_need = colwise ? sh.sc * ((sh.sr + 15) / 16) * (kVarThreads / 64) : sh.nitems;
  const dim3 grid((unsigned)var_wgs(batch, wgs_need), (unsigned)batch);
  hipStream_t s = (hipStream_t)stream;
  if ((variant == NVFP4_VAR_2D || variant == (NVFP4_VAR_2D | NVFP4_VAR_COLWISE)) && n > 0) {
    // 2D without RHT or SR: one launch when the tensors fit on chip
    st = nvfp4host::quantize_2d_onchip(x, batch, rows, cols, colwise, q, sf, g, workspace, s);
    if (st != NVFP4_ENOTSUP) return st;
  }
  uint32_t* partial = (uint32_t*)((char*)workspace + nvfp4host::quantize_2d_onchip_ws_bytes(batch));
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
