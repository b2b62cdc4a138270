// Block-scaled NVFP4 x NVFP4 GEMM on gfx950 MFMA.
//
// NVFP4 serves both weights and activations of MoE expert linears (iwan.kr,
// "NVIDIA shrank GLM-5.2 to 4 bits", section 1); the low-bit operands are
// restored inside the compute kernel instead of being expanded in global
// memory (omidsaffari.com, "LLM quantization guide", section "memory, speed
// and quality").
//
//   C[m][n] = gA * gB * sum_k deq(A)[m][k] * deq(B)[n][k]       (both K-major)
//
// gfx950 has no MFMA that consumes E4M3-per-16 block scales, so every 16-value
// block is dequantized EXACTLY into f16 tiles in LDS: E2M1 * s has at most 6
// significant bits and lies in [2^-10, 2688].  v_cvt_scalef32_pk_f16_fp4 with
// the scale s applies s's power-of-two part (the instruction uses only the
// scale's exponent), and one v_pk_mul_f16 by s's mantissa factor (1 + m/8,
// at most 4 significant bits) finishes the exact product -- about one VALU
// operation per element.  The tiles feed v_mfma_f32_32x32x16_f16 (fp32
// accumulation); gA * gB is applied once in the epilogue.
//
// Tiling: 256 x 256 output per workgroup (the 8192 x 2048 problem is then one
// workgroup per CU), 4 waves of 128 x 128 (4 x 4 MFMA tiles, 256 fp32
// accumulators per lane), K step 64 (4 blocks).  LDS holds two f16 tile
// pairs; while step k is contracted, each thread dequantizes its A row and
// B row of step k+1 into the other pair and step k+2's raw codes load, one
// barrier per step.  When K % 256 == 0 the raw codes are staged in LDS by
// buffer-to-LDS loads and 8 waves of 128 x 64 contract the tile
// (gemm_tile_dma8); otherwise they load into registers (gemm_tile).
#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace nvfp4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GTM = 256, GTN = 256, GTK = 64;
constexpr int GLD = GTK + 8;                 // f16 per LDS row (padding spreads rows over banks)
constexpr int GThreads = 256;

// Raw operand data of one K step for one row: 32 code bytes, 4 scale bytes.
struct RowRaw {
  u32x4 c01, c23;                      // blocks 0,1 and 2,3 (8 bytes each)
  uint32_t s;                          // scale byte of block b in bits 8b..8b+7
};

// One workgroup's rows [r0, r0 + 256) of a K-major NVFP4 operand, addressed
// through buffer resources whose extent ends at the last row: reads of rows
// past the matrix, and reads steered past the extent for K steps at or after
// K, return zeros without a branch and without touching memory (K may be 0,
// with zero-size buffers).  Every load is unconditional, so the compiler
// counts them exactly and the two-steps-ahead prefetch below stays in flight.
struct Operand {
  __amdgpu_buffer_rsrc_t q, s;
  uint32_t qrow, srow;                 // bytes per row: K/2, K/16
};

__device__ __forceinline__ Operand make_operand(const uint8_t* q, const uint8_t* sf, int64_t r0, int64_t rows,
                                                int64_t K) {
  Operand o;
  const int64_t here = rows - r0 < GTM ? rows - r0 : GTM;
  o.qrow = (uint32_t)(K / 2);
  o.srow = (uint32_t)(K / 16);
  o.q = __builtin_amdgcn_make_buffer_rsrc((void*)(q + r0 * (K / 2)), 0, (int)(here * (K / 2)), kBufferWord3);
  o.s = __builtin_amdgcn_make_buffer_rsrc((void*)(sf + r0 * (K / 16)), 0, (int)(here * (K / 16)), kBufferWord3);
  return o;
}

constexpr uint32_t kOutside = 0x80000000u;  // offset beyond every extent (extents stay below 2^31)

// Register operand paths: kRagged (any K % 16 == 0: each block checked on
// its own) and kStep (K % 64 == 0: a step is wholly inside or outside) load
// a thread's raw codes and scale bytes into registers.  K % 256 == 0 stages
// the raw codes in LDS instead (gemm_tile_dma8 below).
constexpr int kRagged = 0, kStep = 1;

template <int kMode>
__device__ __forceinline__ RowRaw load_row(const Operand& o, int lrow, int64_t K, int64_t k0) {
  RowRaw r;
  const bool in = k0 < K;
  const uint32_t qo = in ? (uint32_t)lrow * o.qrow + (uint32_t)(k0 / 2) : kOutside;
  const uint32_t so = in ? (uint32_t)lrow * o.srow + (uint32_t)(k0 / 16) : kOutside;
  if (kMode != kRagged) {              // a step is wholly inside or outside
    r.c01 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(o.q, (int)qo, 0, 0));
    r.c23 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(o.q, (int)(in ? qo + 16 : kOutside), 0, 0));
    r.s = __builtin_amdgcn_raw_buffer_load_b32(o.s, (int)so, 0, 0);
  } else {                             // ragged last step: each block checked on its own
    u32x2 c[4];
    r.s = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const bool bin = k0 + 16 * b < K;
      c[b] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(o.q, (int)(bin ? qo + 8 * b : kOutside), 0, 0));
      r.s |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(o.s, (int)(bin ? so + b : kOutside), 0, 0) << (8 * b);
    }
    r.c01 = u32x4{c[0].x, c[0].y, c[1].x, c[1].y};
    r.c23 = u32x4{c[2].x, c[2].y, c[3].x, c[3].y};
  }
  return r;
}

// Scale words of K steps 4g .. 4g+3 of one row (zeros past K): one
// 16-byte load per 4 steps, so each 128-byte line of scales is fetched from
// L2 a quarter as often as with a 4-byte load per step.
__device__ __forceinline__ u32x4 load_scale_group(const Operand& o, int lrow, int64_t K, int64_t g) {
  const uint32_t so = g * 4 * GTK < K ? (uint32_t)lrow * o.srow + (uint32_t)(g * 16) : kOutside;
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(o.s, (int)so, 0, 0));
}

template <int i>
__device__ __forceinline__ uint32_t word(const u32x4& v) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int sel>
__device__ __forceinline__ f16x2 deq_pair(uint32_t w, float s, f16x2 mf) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, s, sel) * mf;
}

// Dequantizes block b (16 values) of one row exactly into f16 and writes it
// to LDS (dst points at the row).
template <int b>
__device__ __forceinline__ void deq_block_to_lds(const RowRaw& r, _Float16* dst) {
  // s from its E4M3 byte (exact hardware decode, subnormals included)
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)r.s, b);
  // mantissa factor of s in [1, 2): s / 2^floor(log2 s), exact
  const float mfs = __uint_as_float((__float_as_uint(s) & 0x007fffffu) | 0x3f800000u);
  const _Float16 mh = (_Float16)mfs;
  const f16x2 mf = {mh, mh};
  const uint32_t cx = b == 0 ? r.c01.x : b == 1 ? r.c01.z : b == 2 ? r.c23.x : r.c23.z;
  const uint32_t cy = b == 0 ? r.c01.y : b == 1 ? r.c01.w : b == 2 ? r.c23.y : r.c23.w;
  f16x8 lo, hi;
  f16x2 p;
  p = deq_pair<0>(cx, s, mf); lo[0] = p.x; lo[1] = p.y;
  p = deq_pair<1>(cx, s, mf); lo[2] = p.x; lo[3] = p.y;
  p = deq_pair<2>(cx, s, mf); lo[4] = p.x; lo[5] = p.y;
  p = deq_pair<3>(cx, s, mf); lo[6] = p.x; lo[7] = p.y;
  p = deq_pair<0>(cy, s, mf); hi[0] = p.x; hi[1] = p.y;
  p = deq_pair<1>(cy, s, mf); hi[2] = p.x; hi[3] = p.y;
  p = deq_pair<2>(cy, s, mf); hi[4] = p.x; hi[5] = p.y;
  p = deq_pair<3>(cy, s, mf); hi[6] = p.x; hi[7] = p.y;
  *(f16x8*)(dst + 16 * b) = lo;
  *(f16x8*)(dst + 16 * b + 8) = hi;
}

// One 16-wide k substep: 16 MFMAs on the fragments in a/b while the next
// substep's fragments load from LDS and block kk of the next K step is
// dequantized into the other LDS buffer.  The scheduling groups interleave
// one MFMA with a few VALU and LDS instructions, so the single wave on each
// SIMD keeps its matrix core fed while it does the dequantization.
template <int kk>
__device__ __forceinline__ void substep(f32x16 (&acc)[4][4], f16x8 (&a)[4], f16x8 (&b)[4], const _Float16* Acur,
                                        const _Float16* Bcur, const RowRaw& ra, const RowRaw& rb, _Float16* Anext,
                                        _Float16* Bnext) {
  static_assert(kk < 3, "the last substep is substep_last");
  __builtin_amdgcn_sched_barrier(0);               // each substep is its own scheduling region
  f16x8 an[4], bn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) an[i] = *(const f16x8*)(Acur + i * 32 * GLD + 16 * (kk + 1));
#pragma unroll
  for (int j = 0; j < 4; ++j) bn[j] = *(const f16x8*)(Bcur + j * 32 * GLD + 16 * (kk + 1));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
  deq_block_to_lds<kk>(ra, Anext);
  deq_block_to_lds<kk>(rb, Bnext);
  // 16 MFMA; about 40 VALU; 8 LDS reads and 4 LDS writes
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);     // VALU
    if (m < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    else if (m < 12) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = an[i]; b[i] = bn[i]; }
}

// The last substep of a K step.  Its 16 MFMAs are split around the
// workgroup barrier that ends the step: the first 8 run while block 3 of the
// next step is dequantized into the other buffer; after the barrier (the
// other buffer is complete and the current one is no longer read) the
// fragments of the next step's first substep are read while the last 8 run,
// so the LDS latency after the barrier is hidden behind MFMAs.
__device__ __forceinline__ void substep_last(f32x16 (&acc)[4][4], f16x8 (&a)[4], f16x8 (&b)[4], const _Float16* Anb,
                                             const _Float16* Bnb, const RowRaw& ra, const RowRaw& rb,
                                             _Float16* Anext, _Float16* Bnext) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
  deq_block_to_lds<3>(ra, Anext);
  deq_block_to_lds<3>(rb, Bnext);
  // 8 MFMA; about 40 VALU; 4 LDS writes
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);     // VALU
    if (m >= 4) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
  }
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
  f16x8 an[4], bn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) an[i] = *(const f16x8*)(Anb + i * 32 * GLD);
#pragma unroll
  for (int j = 0; j < 4; ++j) bn[j] = *(const f16x8*)(Bnb + j * 32 * GLD);
#pragma unroll
  for (int i = 2; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = an[i]; b[i] = bn[i]; }
}

// One 256 x 256 output tile: rows [m0, m_end) of A (K-major NVFP4, at most
// 256 of them) against rows [n0, n_end) of B, C row stride ldc, scaled by
// gab in the epilogue.  As / Bs are the workgroup's LDS tiles.
template <int kMode>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ aq, const uint8_t* __restrict__ asf,
                                          int64_t m0, int64_t m_end, const uint8_t* __restrict__ bq,
                                          const uint8_t* __restrict__ bsf, int64_t n0, int64_t n_end, int64_t K,
                                          float gab, float* __restrict__ C, int64_t ldc,
                                          _Float16 (*As)[GTM][GLD], _Float16 (*Bs)[GTN][GLD]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;       // 2 x 2 waves of 128 x 128
  const Operand A = make_operand(aq, asf, m0, m_end, K), B = make_operand(bq, bsf, n0, n_end, K);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Software pipeline over K steps: while the MFMAs of step k read LDS buffer
  // k%2, each thread dequantizes its A row and B row of step k+1 into the
  // other buffer (one block per substep) and the raw codes of step k+2 load.
  // Steps past the last one read zeros and write an unread buffer.
  const int64_t nk = (K + GTK - 1) / GTK;
  RowRaw ra = load_row<kMode>(A, tid, K, 0);
  RowRaw rb = load_row<kMode>(B, tid, K, 0);
  deq_block_to_lds<0>(ra, &As[0][tid][0]);
  deq_block_to_lds<1>(ra, &As[0][tid][0]);
  deq_block_to_lds<2>(ra, &As[0][tid][0]);
  deq_block_to_lds<3>(ra, &As[0][tid][0]);
  deq_block_to_lds<0>(rb, &Bs[0][tid][0]);
  deq_block_to_lds<1>(rb, &Bs[0][tid][0]);
  deq_block_to_lds<2>(rb, &Bs[0][tid][0]);
  deq_block_to_lds<3>(rb, &Bs[0][tid][0]);
  ra = load_row<kMode>(A, tid, K, GTK);
  rb = load_row<kMode>(B, tid, K, GTK);
  __syncthreads();
  const int arow = wm * 128 + (lane & 31), brow = wn * 128 + (lane & 31), kof = 8 * (lane >> 5);
  // fragments of step 0's first substep; later steps' are read by substep_last
  f16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = *(const f16x8*)(&As[0][arow][kof] + i * 32 * GLD);
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = *(const f16x8*)(&Bs[0][brow][kof] + j * 32 * GLD);
  // iteration kt contracts step kt, dequantizes step kt+1 and loads step kt+2
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    const RowRaw ra2 = load_row<kMode>(A, tid, K, (kt + 2) * GTK);
    const RowRaw rb2 = load_row<kMode>(B, tid, K, (kt + 2) * GTK);
    const _Float16* Acur = &As[buf][arow][kof];
    const _Float16* Bcur = &Bs[buf][brow][kof];
    _Float16* An = &As[buf ^ 1][tid][0];
    _Float16* Bn = &Bs[buf ^ 1][tid][0];
    substep<0>(acc, a, b, Acur, Bcur, ra, rb, An, Bn);
    substep<1>(acc, a, b, Acur, Bcur, ra, rb, An, Bn);
    substep<2>(acc, a, b, Acur, Bcur, ra, rb, An, Bn);
    substep_last(acc, a, b, &As[buf ^ 1][arow][kof], &Bs[buf ^ 1][brow][kof], ra, rb, An, Bn);
    ra = ra2;
    rb = rb2;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
        if (row < m_end && col < n_end) C[row * ldc + col] = acc[i][j][e] * gab;
      }
}

// ------------------------------------------------------------ K % 256 == 0: raw codes through LDS
// 8 waves of 128 x 64 (2 x 4) run two waves per SIMD, so one wave's
// dequantization, LDS traffic and barrier wait overlap the other's MFMAs.
// Thread t dequantizes one row: A row t for t < 256, else B row t - 256.
//
// The raw codes of a K step reach LDS by buffer-to-LDS loads, which hold no
// VGPRs and skip the register return path; the scale words of 4 steps come
// in one 16-byte register load per row.  Each wave loads exactly the raw rows
// its own threads dequantize (thread t's 32 bytes at raw + 32 t), so one raw
// buffer suffices: a wave's next load is issued only after its own reads of
// the buffer have returned, with no workgroup barrier involved.  Half h of
// raw row t sits at half position h ^ ((t >> 2 ^ t >> 3) & 1), which puts 8
// (and 16) consecutive rows' reads on distinct banks.  The f16 tiles keep
// the 72-half row padding of gemm_tile (conflict-free reads and writes).
constexpr int GThreads8 = 512;

struct GemmDmaSmem {
  _Float16 af[2][GTM][GLD];
  _Float16 bf[2][GTN][GLD];
  uint8_t raw[2 * GTM * 32];
};
static_assert(sizeof(GemmDmaSmem) <= 160 * 1024, "LDS budget");

typedef __attribute__((address_space(3))) void gemm_lds_t;

__device__ __forceinline__ int raw_swz(int t) { return ((t >> 2) ^ (t >> 3)) & 1; }

// Wave w's raw rows of the step at k0: rows t = 64 w .. 64 w + 63 of the raw
// buffer (operand rows t & 255 of A for w < 4, of B otherwise), 32 rows
// (1 KiB) per instruction.
__device__ __forceinline__ void dma_codes8(const Operand& o, int wave, int lane, int64_t k0, uint8_t* raw) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t0 = 64 * wave + 32 * j, t = t0 + (lane >> 1);
    const int h = (lane & 1) ^ raw_swz(t);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(o.q, (gemm_lds_t*)(raw + t0 * 32), 16,
                                             (uint32_t)(t & 255) * o.qrow + (uint32_t)(k0 / 2) + 16u * h, 0, 0, 0);
  }
}

// Raw row t's 32 code bytes from LDS (both halves, in order).
__device__ __forceinline__ void read_codes(const uint8_t* raw, int t, RowRaw& out) {
  const int sz = raw_swz(t);
  out.c01 = *(const u32x4*)(raw + t * 32 + 16 * sz);
  out.c23 = *(const u32x4*)(raw + t * 32 + 16 * (sz ^ 1));
}

__device__ __forceinline__ void wait_vm0() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));   // vmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0x3F | (0x3 << 14));   // lgkmcnt(0), vmcnt at its maximum
  __builtin_amdgcn_sched_barrier(0);
}

template <int kk>
__device__ __forceinline__ void dma8_substep(f32x16 (&acc)[4][2], f16x8 (&a)[4], f16x8 (&b)[2], const _Float16* Acur,
                                             const _Float16* Bcur, const RowRaw& rr, _Float16* Dn) {
  __builtin_amdgcn_sched_barrier(0);
  // raised wave priority while the substep's MFMAs issue (the other wave of
  // the SIMD yields the issue slot): 0.1914 -> 0.1897 ms and the grouped
  // GEMM 3.266 -> 3.222 ms in one run, consistent over three runs; raising
  // it for the barrier substep as well gained nothing
  __builtin_amdgcn_s_setprio(1);
  f16x8 an[4], bn[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) an[i] = *(const f16x8*)(Acur + i * 32 * GLD + 16 * (kk + 1));
#pragma unroll
  for (int j = 0; j < 2; ++j) bn[j] = *(const f16x8*)(Bcur + j * 32 * GLD + 16 * (kk + 1));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
  deq_block_to_lds<kk>(rr, Dn);
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);     // VALU
    if (m < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
    else __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);         // DS write
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = an[i];
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = bn[j];
}

// Iteration kt contracts step kt (tile kt % 2), dequantizes step kt+1 from
// its raw codes (in registers since the end of iteration kt-1) into the
// other tile, and loads step kt+2's raw codes (issued after the first
// substep, when the wave's reads of the raw buffer have returned; waited
// for at the end of the iteration and read back after its barrier).
__device__ __forceinline__ void gemm_tile_dma8(const uint8_t* __restrict__ aq, const uint8_t* __restrict__ asf,
                                               int64_t m0, int64_t m_end, const uint8_t* __restrict__ bq,
                                               const uint8_t* __restrict__ bsf, int64_t n0, int64_t n_end, int64_t K,
                                               float gab, float* __restrict__ C, int64_t ldc, GemmDmaSmem& sm) {
  const int tid = threadIdx.x;
  const int wave = wave_id(), lane = tid & 63;    // wave index in an SGPR (the loads' LDS base)
  const int wm = wave >> 2, wn = wave & 3;        // 2 x 4 waves of 128 x 64
  const Operand A = make_operand(aq, asf, m0, m_end, K), B = make_operand(bq, bsf, n0, n_end, K);
  const bool isb = wave >= 4;                     // this wave dequantizes (and loads) B rows
  const Operand& X = isb ? B : A;
  const int row = tid & 255;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int64_t nk = K / GTK;                      // K % 256 == 0, so nk % 4 == 0
  u32x4 s_cur = load_scale_group(X, row, K, 0), s_nxt = load_scale_group(X, row, K, 1);
  _Float16* const x0 = isb ? &sm.bf[0][row][0] : &sm.af[0][row][0];
  _Float16* const x1 = isb ? &sm.bf[1][row][0] : &sm.af[1][row][0];
  // step 0's codes straight into registers and step 1's into the raw buffer,
  // both in flight at once (one memory round trip before the loop, not two)
  RowRaw rr;
  {
    const uint32_t qo = (uint32_t)row * X.qrow;
    rr.c01 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(X.q, (int)qo, 0, 0));
    rr.c23 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(X.q, (int)(qo + 16), 0, 0));
  }
  dma_codes8(X, wave, lane, GTK, sm.raw);
  wait_vm0();
  rr.s = s_cur.x;
  deq_block_to_lds<0>(rr, x0);
  deq_block_to_lds<1>(rr, x0);
  deq_block_to_lds<2>(rr, x0);
  deq_block_to_lds<3>(rr, x0);
  read_codes(sm.raw, tid, rr);
  __syncthreads();                                 // tile 0 complete
  const int arow = wm * 128 + (lane & 31), brow = wn * 64 + (lane & 31), kof = 8 * (lane >> 5);
  f16x8 a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = *(const f16x8*)(&sm.af[0][arow][kof] + i * 32 * GLD);
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = *(const f16x8*)(&sm.bf[0][brow][kof] + j * 32 * GLD);
  auto iteration = [&](int64_t kt, auto U) {
    constexpr int u = decltype(U)::value;          // kt % 4
    const int buf = (int)(kt & 1);
    if ((u + 1) % 4 == 0) {                        // step kt+1 opens group (kt+1)/4
      s_cur = s_nxt;
      s_nxt = load_scale_group(X, row, K, (kt + 1) / 4 + 1);
    }
    rr.s = word<(u + 1) % 4>(s_cur);
    const _Float16* Acur = &sm.af[buf][arow][kof];
    const _Float16* Bcur = &sm.bf[buf][brow][kof];
    _Float16* Dn = buf ? x0 : x1;
    dma8_substep<0>(acc, a, b, Acur, Bcur, rr, Dn);
    if (kt + 2 < nk) {
      wait_lgkm0();                                // this wave's reads of the raw buffer have returned
      dma_codes8(X, wave, lane, (kt + 2) * GTK, sm.raw);
    }
    dma8_substep<1>(acc, a, b, Acur, Bcur, rr, Dn);
    dma8_substep<2>(acc, a, b, Acur, Bcur, rr, Dn);
    // last substep: 4 MFMAs with block 3's dequantization, the barrier, then
    // the next step's first fragments and step kt+2's raw codes are read
    // under the other 4 MFMAs
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    deq_block_to_lds<3>(rr, Dn);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // VALU
      if (m >= 2) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vm0();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    f16x8 an[4], bn[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) an[i] = *(const f16x8*)(&sm.af[buf ^ 1][arow][kof] + i * 32 * GLD);
#pragma unroll
    for (int j = 0; j < 2; ++j) bn[j] = *(const f16x8*)(&sm.bf[buf ^ 1][brow][kof] + j * 32 * GLD);
    read_codes(sm.raw, tid, rr);
#pragma unroll
    for (int i = 2; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = an[i];
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = bn[j];
  };
  for (int64_t kt = 0; kt < nk; kt += 4) {
    iteration(kt, std::integral_constant<int, 0>());
    iteration(kt + 1, std::integral_constant<int, 1>());
    iteration(kt + 2, std::integral_constant<int, 2>());
    iteration(kt + 3, std::integral_constant<int, 3>());
  }
  // Epilogue.  C layout of the 32 x 32 MFMA: lane l, element e is row
  // 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32.
  if (m0 + GTM <= m_end && n0 + GTN <= n_end && ldc <= (1 << 20)) {
    // Whole tile: a buffer resource from the tile's first element and 32-bit
    // offsets (256 rows of at most 2^20 floats stay below 2^30 bytes).  Each
    // accumulator's row offset is uniform, so the only per-element vector
    // work is the gA * gB product; with 64-bit addresses and per-element
    // bounds checks the epilogue ran about 900 vector instructions per wave.
    // Each store writes two whole 128-byte lines of C, which is written once:
    // non-temporal.
    const int ld = (int)ldc;
    const __amdgpu_buffer_rsrc_t cr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(C + m0 * ldc + n0), 0, GTM * ld * 4, kBufferWord3);
    const int vo = ((wm * 128 + 4 * (lane >> 5)) * ld + wn * 64 + (lane & 31)) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int so = (i * 32 + 8 * (e >> 2) + (e & 3)) * ld * 4;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][e] * gab), cr, vo + j * 128, so,
                                                kStreamLoad);
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t r = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int64_t c = n0 + wn * 64 + j * 32 + (lane & 31);
        if (r < m_end && c < n_end) C[r * ldc + c] = acc[i][j][e] * gab;
      }
}

__global__ void __launch_bounds__(GThreads8) gemm8_kernel(const uint8_t* __restrict__ aq,
                                                          const uint8_t* __restrict__ asf,
                                                          const float* __restrict__ ag, const uint8_t* __restrict__ bq,
                                                          const uint8_t* __restrict__ bsf,
                                                          const float* __restrict__ bg, int64_t M, int64_t N,
                                                          int64_t K, float* __restrict__ C) {
  const int64_t tile = xcd_tile((int64_t)blockIdx.y * gridDim.x + blockIdx.x, (int64_t)gridDim.x * gridDim.y);
  const int64_t m0 = tile / gridDim.x * GTM, n0 = tile % gridDim.x * GTN;
  __shared__ __attribute__((aligned(16))) GemmDmaSmem sm;
  gemm_tile_dma8(aq, asf, m0, M, bq, bsf, n0, N, K, ag[0] * bg[0], C, N, sm);
}

template <int kMode>
__global__ void __launch_bounds__(GThreads) gemm_kernel(const uint8_t* __restrict__ aq, const uint8_t* __restrict__ asf,
                                                        const float* __restrict__ ag, const uint8_t* __restrict__ bq,
                                                        const uint8_t* __restrict__ bsf, const float* __restrict__ bg,
                                                        int64_t M, int64_t N, int64_t K, float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][GTM][GLD];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][GTN][GLD];
  const int64_t tile = xcd_tile((int64_t)blockIdx.y * gridDim.x + blockIdx.x, (int64_t)gridDim.x * gridDim.y);
  const int64_t m0 = tile / gridDim.x * GTM, n0 = tile % gridDim.x * GTN;
  gemm_tile<kMode>(aq, asf, m0, M, bq, bsf, n0, N, K, ag[0] * bg[0], C, N, As, Bs);
}

// Grouped GEMM: rows of A are grouped by expert, rows [off[e], off[e+1])
// multiplying expert e's weight B_e = b[e] ([N][K]).  grid.y enumerates the
// (expert, 256-row tile) pairs in expert order; a workgroup finds its pair by
// walking the offsets (clamped to [0, M], so inconsistent offsets never
// reach outside A or C) and exits when its index is past the last tile.
__device__ __forceinline__ bool grouped_tile(const int32_t* __restrict__ off, int experts, int64_t M, int& e,
                                             int64_t& m0, int64_t& hi) {
  int64_t tile = blockIdx.y;
  int64_t lo = 0;
  hi = 0;
  for (e = 0; e < experts; ++e) {
    lo = off[e] < 0 ? 0 : (off[e] > M ? M : off[e]);
    hi = off[e + 1] < lo ? lo : (off[e + 1] > M ? M : off[e + 1]);
    const int64_t tiles = (hi - lo + GTM - 1) / GTM;
    if (tile < tiles) break;
    tile -= tiles;
  }
  m0 = lo + tile * GTM;
  return e < experts;                                  // false: past the last tile, no work
}

template <int kMode>
__global__ void __launch_bounds__(GThreads) grouped_gemm_kernel(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ asf, const float* __restrict__ ag,
    const uint8_t* __restrict__ bq, const uint8_t* __restrict__ bsf, const float* __restrict__ bg,
    const int32_t* __restrict__ off, int experts, int64_t M, int64_t N, int64_t K, float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][GTM][GLD];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][GTN][GLD];
  int e;
  int64_t m0, hi;
  if (!grouped_tile(off, experts, M, e, m0, hi)) return;
  const int64_t n0 = (int64_t)blockIdx.x * GTN;
  const int64_t wq = N * (K / 2), ws = N * (K / 16);   // bytes per expert weight, scales
  gemm_tile<kMode>(aq, asf, m0, hi, bq + e * wq, bsf + e * ws, n0, N, K, ag[0] * bg[e], C, N, As, Bs);
}

__global__ void __launch_bounds__(GThreads8) grouped_gemm8_kernel(
    const uint8_t* __restrict__ aq, const uint8_t* __restrict__ asf, const float* __restrict__ ag,
    const uint8_t* __restrict__ bq, const uint8_t* __restrict__ bsf, const float* __restrict__ bg,
    const int32_t* __restrict__ off, int experts, int64_t M, int64_t N, int64_t K, float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) GemmDmaSmem sm;
  int e;
  int64_t m0, hi;
  if (!grouped_tile(off, experts, M, e, m0, hi)) return;
  const int64_t n0 = (int64_t)blockIdx.x * GTN;
  const int64_t wq = N * (K / 2), ws = N * (K / 16);
  gemm_tile_dma8(aq, asf, m0, hi, bq + e * wq, bsf + e * ws, n0, N, K, ag[0] * bg[e], C, N, sm);
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
  if ((M + GTM - 1) / GTM > 65535 || (N + GTN - 1) / GTN > 2147483647LL) return NVFP4_EINVAL;
  // a workgroup's 256-row operand slab is addressed with 32-bit offsets
  if (K > (1LL << 22)) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(a_q) || !nvfp4host::aligned16(b_q) || !nvfp4host::aligned16(c)) return NVFP4_EALIGN;
  if ((reinterpret_cast<uintptr_t>(a_g) & 3u) || (reinterpret_cast<uintptr_t>(b_g) & 3u)) return NVFP4_EALIGN;
  nvfp4_status st = nvfp4host::check_device();
  if (st) return st;
  const dim3 grid((unsigned)((N + GTN - 1) / GTN), (unsigned)((M + GTM - 1) / GTM));
  // whole-step paths: K a multiple of 64 (of 256 for grouped scale loads)
  // and 16-byte aligned scale bases, so scale rows are 4- (16-) byte aligned
  const bool aligned = K % GTK == 0 && nvfp4host::aligned16(a_sf) && nvfp4host::aligned16(b_sf);
  hipStream_t s = (hipStream_t)stream;
  if (aligned && K % (4 * GTK) == 0)
    gemm8_kernel<<<grid, GThreads8, 0, s>>>(a_q, a_sf, a_g, b_q, b_sf, b_g, M, N, K, c);
  else if (aligned)
    gemm_kernel<kStep><<<grid, GThreads, 0, s>>>(a_q, a_sf, a_g, b_q, b_sf, b_g, M, N, K, c);
  else
    gemm_kernel<kRagged><<<grid, GThreads, 0, s>>>(a_q, a_sf, a_g, b_q, b_sf, b_g, M, N, K, c);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

extern "C" nvfp4_status nvfp4_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sf, const float* a_g,
                                           const uint8_t* b_q, const uint8_t* b_sf, const float* b_g,
                                           const int32_t* offsets, int32_t experts, int64_t M, int64_t N, int64_t K,
                                           float* c, void* stream) {
  using namespace nvfp4;
  if (experts <= 0 || M < 0 || N < 0 || K < 0 || K % kBlock) return NVFP4_EINVAL;
  if (M == 0 || N == 0) return NVFP4_OK;
  if (!a_g || !b_g || !c || !offsets) return NVFP4_EINVAL;
  if (K > 0 && (!a_q || !a_sf || !b_q || !b_sf)) return NVFP4_EINVAL;
  // upper bound on the (expert, row tile) pairs: every expert adds at most one partial tile
  const int64_t tiles_y = (M + GTM - 1) / GTM + experts;
  if (tiles_y > 65535 || (N + GTN - 1) / GTN > 2147483647LL) return NVFP4_EINVAL;
  if (K > (1LL << 22)) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(a_q) || !nvfp4host::aligned16(b_q) || !nvfp4host::aligned16(c)) return NVFP4_EALIGN;
  if ((reinterpret_cast<uintptr_t>(a_g) & 3u) || (reinterpret_cast<uintptr_t>(b_g) & 3u) ||
      (reinterpret_cast<uintptr_t>(offsets) & 3u))
    return NVFP4_EALIGN;
  nvfp4_status st = nvfp4host::check_device();
  if (st) return st;
  const dim3 grid((unsigned)((N + GTN - 1) / GTN), (unsigned)tiles_y);
  // aligned path as for nvfp4_gemm; each expert's weight starts at a multiple
  // of N*K/2 code bytes and N*K/16 scale bytes, aligned with K % 64 == 0
  const bool aligned = K % GTK == 0 && nvfp4host::aligned16(a_sf) && nvfp4host::aligned16(b_sf);
  hipStream_t s = (hipStream_t)stream;
  if (aligned && K % (4 * GTK) == 0)
    grouped_gemm8_kernel<<<grid, GThreads8, 0, s>>>(a_q, a_sf, a_g, b_q, b_sf, b_g, offsets, experts, M, N, K, c);
  else if (aligned)
    grouped_gemm_kernel<kStep><<<grid, GThreads, 0, s>>>(a_q, a_sf, a_g, b_q, b_sf, b_g, offsets, experts, M, N, K, c);
  else
    grouped_gemm_kernel<kRagged><<<grid, GThreads, 0, s>>>(a_q, a_sf, a_g, b_q, b_sf, b_g, offsets, experts, M, N, K,
                                                           c);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}
