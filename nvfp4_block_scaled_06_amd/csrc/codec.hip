// Quantize / dequantize kernels and their C-ABI entry points.
//
// Two-level microscaling (axbrief.com, "NVFP4: how NVIDIA pre-trained a 12B
// model on 10 trillion tokens", section "E2M1 format and two-level scaling"):
// a tensor amax pass (the FP32 tensor scale sets the overall range), then an
// encode pass that derives each 16-value block's E4M3 scale from the block's
// amax and rounds every element onto the E2M1 grid, two codes per byte.
// Dequantization restores values from the scales (omidsaffari.com, "LLM
// quantization guide", section "What is LLM quantization").
//
// Memory layout per tensor: a flat run of 16-value blocks (cols % 16 == 0,
// so rows never split a block).  Kernels work in HALF blocks: half block h
// is 16 bytes of bf16 at x + 16h, 4 code bytes at q + 4h, and shares the
// scale byte sf[h/2] with its partner.  Lane i of a wave takes half block
// base+i, so each load / store instruction covers one contiguous run.
//
// Launch modes of nvfp4_quantize:
//  TWO_KERNEL  amax_partial_kernel (per-workgroup maxima, no atomics) then
//              encode_kernel (reduces the partials, builds the table, encodes).
//  FUSED       one cooperative launch whose workgroups walk the batch
//              tensor by tensor.  fused_onchip_kernel when a tensor fits on
//              chip (registers + LDS of the whole GPU): every input byte is
//              read from HBM once.  Otherwise fused_quantize_kernel: each
//              workgroup reduces its slice of tensor t, publishes it
//              (agent-scope atomics), then encodes its slice of tensor t-1,
//              read again newest-first.
#include <algorithm>

#include "common.hpp"

namespace nvfp4 {

constexpr int kU = 4;   // half blocks per lane per loop trip (loads in flight)

// ------------------------------------------------------------ pass 1: amax
// grid (P, batch): workgroup p of tensor t reduces a strided share of the
// tensor's 16-byte vectors into partial[t*P + p] (bf16 magnitude bits).
__global__ void __launch_bounds__(kThreads) amax_partial_kernel(const u32x4* __restrict__ x, int64_t vec_per_tensor,
                                                                uint32_t* __restrict__ partial) {
  const int t = blockIdx.y;
  const u32x4* xt = x + (int64_t)t * vec_per_tensor;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t m0 = 0, m1 = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < vec_per_tensor; i += 4 * stride) {
    const u32x4 a = xt[i], b = xt[i + stride], c = xt[i + 2 * stride], d = xt[i + 3 * stride];
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

// ------------------------------------------------------------ encode pieces
// Per-tensor state of the encode pass: g, the reciprocal of d6 = RN32(6g) and
// the fp64 reciprocal of every block divisor d = RN32(s g) in LDS.
__device__ __forceinline__ void build_table(double* table, float g) {
  for (uint32_t j = threadIdx.x; j < 127u; j += blockDim.x) table[j] = recip_entry(j, g);
}

// Encodes one wave chunk of half blocks [base, base+64) clipped to [lo, hi)
// (the ragged tail of a tensor or slice).  All lanes run it together, so the
// DPP pair exchange is always well defined.
__device__ __forceinline__ void encode_tail(const u32x4* __restrict__ xt, uint32_t* __restrict__ qt,
                                            uint8_t* __restrict__ st, int64_t base, int64_t lo, int64_t hi,
                                            double r6, const double* table) {
  const int lane = threadIdx.x & 63;
  const int64_t hb = base + lane;
  const bool ok = hb >= lo && hb < hi;
  const u32x4 v = ok ? __builtin_nontemporal_load(xt + hb) : u32x4{0u, 0u, 0u, 0u};
  const uint32_t sbyte = block_scale_byte(pair_max(half_absmax_bits(v)), r6);
  const uint32_t code = encode_half(v, table[sbyte]);
  if (ok) {
    qt[hb] = code;
    if ((lane & 1) == 0) st[hb >> 1] = (uint8_t)sbyte;
  }
}

// Encodes kU whole wave chunks (64 half blocks each, every one in range):
// chunk u starts at half block c[u] (wave-uniform, a multiple of 64).  No
// bounds checks: the loads and stores use a scalar base plus the lane offset.
__device__ __forceinline__ void encode_chunks(const u32x4* __restrict__ xt, uint32_t* __restrict__ qt,
                                              uint8_t* __restrict__ st, const int64_t (&c)[kU], double r6,
                                              const double* table) {
  const int lane = threadIdx.x & 63;
  u32x4 v[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load((xt + c[u]) + lane);   // last use of x
  uint32_t sbyte[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) sbyte[u] = block_scale_byte(pair_max(half_absmax_bits(v[u])), r6);
  double r[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) r[u] = table[sbyte[u]];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const uint32_t code = encode_half(v[u], r[u]);
    __builtin_nontemporal_store(code, (qt + c[u]) + lane);
    if ((lane & 1) == 0) (st + c[u] / 2)[lane >> 1] = (uint8_t)sbyte[u];
  }
}

// ------------------------------------------------------------ pass 2 (two-kernel) / with_scale
// grid (P, batch).  kFromPartials: g = RN32(amax/2688) from pass-1 partials;
// otherwise g is read from gin[t] (quantize_with_scale).
template <bool kFromPartials>
__global__ void __launch_bounds__(kThreads) encode_kernel(const u32x4* __restrict__ x, int64_t hb_per_tensor,
                                                          const uint32_t* __restrict__ partial, int npartial,
                                                          const float* __restrict__ gin, float* __restrict__ gout,
                                                          uint32_t* __restrict__ q, uint8_t* __restrict__ sf) {
  // Tensors and chunks are walked in the reverse of pass 1's order, so the
  // most recently read data -- still in the Infinity Cache -- is encoded first.
  const int t = gridDim.y - 1 - blockIdx.y;
  __shared__ double table[128];
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
  const double r6 = recip_d6(g);
  build_table(table, g);
  __syncthreads();
  const int64_t off = (int64_t)t * hb_per_tensor;
  const u32x4* xt = x + off;
  uint32_t* qt = q + off;
  uint8_t* st = sf + off / 2;
  // whole 64-half-block chunks, kU per wave per trip, then the ragged rest
  const int64_t nwaves = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t gw = (int64_t)blockIdx.x * (kThreads / 64) + wave_id();
  const int64_t nchunks = (hb_per_tensor + 63) / 64;
  const int64_t nfull = hb_per_tensor / 64;
  if (gw == 0 && nfull < nchunks)                      // ragged last chunk first
    encode_tail(xt, qt, st, nfull * 64, 0, hb_per_tensor, r6, table);
  // chunk index counted from the end: j = nfull - 1 - k
  int64_t k = gw;
  for (; k + (kU - 1) * nwaves < nfull; k += kU * nwaves) {
    int64_t c[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) c[u] = (nfull - 1 - (k + u * nwaves)) * 64;
    encode_chunks(xt, qt, st, c, r6, table);
  }
  for (; k < nfull; k += nwaves) encode_tail(xt, qt, st, (nfull - 1 - k) * 64, 0, hb_per_tensor, r6, table);
}

// ------------------------------------------------------------ fused persistent launch
// Workspace header (zero-filled by the caller once; the kernel's last
// workgroup restores it to zero).  Per tensor there is one 64-byte line per
// arrival group {arrive, amax, go} and one top line {arrive, amax}: workgroup
// w belongs to group w % kGroups, so no counter sees more than ~G/kGroups
// atomics per tensor (same-address atomics serialize at the coherence point).
constexpr int kGroups = 32;
constexpr size_t kFusedHeaderBytes = 256;
constexpr size_t kLineWords = 16;                      // 64-byte lines
constexpr size_t kTensorWords = (kGroups + 1) * kLineWords;
constexpr uint32_t kSpinLimit = 1u << 24;              // ~seconds: only a non-resident grid gets there

struct FusedHeader {
  uint32_t done;
  uint32_t error;
};

__device__ __forceinline__ uint32_t* fused_line(uint32_t* ws, int t, int line) {
  return ws + kFusedHeaderBytes / 4 + (size_t)t * kTensorWords + (size_t)line * kLineWords;
}

// Publishes this workgroup's maximum m of tensor t (thread 0 only).
// Only atomic locations carry data between workgroups (the input is read-only
// and outputs are not read back), so relaxed agent-scope atomics suffice;
// acquire/release would write back and invalidate the whole L2 every time.
// Each arrival is made data-dependent on the returned old maximum (always
// < 2^15), so it is issued only after the maximum has been performed.
__device__ __forceinline__ void fused_arrive(uint32_t* ws, int t, uint32_t m, int G) {
  const int grp = blockIdx.x % kGroups;
  const uint32_t members = (uint32_t)((G - grp + kGroups - 1) / kGroups);
  const uint32_t ngroups = (uint32_t)(G < kGroups ? G : kGroups);
  uint32_t* gl = fused_line(ws, t, grp);
  const uint32_t om = __hip_atomic_fetch_max(gl + 1, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t oa = __hip_atomic_fetch_add(gl, 1u + (om >> 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (oa + 1 != members) return;
  // last of its group: every member's maximum is in gl[1] (their arrivals,
  // which follow their maxima, have all been counted)
  const uint32_t gm = __hip_atomic_load(gl + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t* top = fused_line(ws, t, kGroups);
  const uint32_t om2 = __hip_atomic_fetch_max(top + 1, gm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t oa2 = __hip_atomic_fetch_add(top, 1u + (om2 >> 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (oa2 + 1 != ngroups) return;
  // last group overall: release every group's waiters
  const uint32_t tm = __hip_atomic_load(top + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (uint32_t k = 0; k < ngroups; ++k)
    __hip_atomic_store(fused_line(ws, t, (int)k) + 2, 0x80000000u | tm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits (thread 0 only) until tensor t's maximum is published to this
// workgroup's group; returns it with bit 31 set, or 0 after the spin limit.
__device__ __forceinline__ uint32_t fused_wait(uint32_t* ws, int t) {
  uint32_t* go = fused_line(ws, t, blockIdx.x % kGroups) + 2;
  for (uint32_t it = 0; it < kSpinLimit; ++it) {
    const uint32_t v = __hip_atomic_load(go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v & 0x80000000u) return v;
    __builtin_amdgcn_s_sleep(2);
  }
  __hip_atomic_store(&((FusedHeader*)ws)->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 0u;
}

__global__ void __launch_bounds__(kThreads) fused_quantize_kernel(const u32x4* __restrict__ x, int batch,
                                                                  int64_t hb_per_tensor, uint32_t* ws,
                                                                  float* __restrict__ gout, uint32_t* __restrict__ q,
                                                                  uint8_t* __restrict__ sf) {
  __shared__ double table[128];
  __shared__ uint32_t red[kThreads / 64];
  __shared__ uint32_t sh_amax;
  __shared__ uint32_t sh_last;
  const int G = gridDim.x, w = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  // this workgroup's contiguous slice of every tensor, in whole waves
  const int64_t chunk = ((hb_per_tensor + G - 1) / G + 63) & ~(int64_t)63;
  const int64_t lo = std::min<int64_t>((int64_t)w * chunk, hb_per_tensor);
  const int64_t hi = std::min<int64_t>(lo + chunk, hb_per_tensor);
  const int64_t step = kThreads;                       // the workgroup's waves tile 256 half blocks

  for (int t = 0; t <= batch; ++t) {
    if (t < batch) {                                   // pass 1 on tensor t
      const u32x4* xt = x + (int64_t)t * hb_per_tensor;
      uint32_t m0 = 0, m1 = 0;
      int64_t i = lo + threadIdx.x;
      for (; i + step < hi; i += 2 * step) {
        const u32x4 a = xt[i], b = xt[i + step];
        m0 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m0, a.x), a.y), a.z), a.w);
        m1 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m1, b.x), b.y), b.z), b.w);
      }
      if (i < hi) {
        const u32x4 a = xt[i];
        m0 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m0, a.x), a.y), a.z), a.w);
      }
      uint32_t m = wave_max_u32(halves_max(pk_absmax(m0, m1)));
      if ((threadIdx.x & 63) == 0) red[wave] = m;
      __syncthreads();
      if (threadIdx.x == 0) {
        uint32_t r = red[0];
#pragma unroll
        for (int k = 1; k < kThreads / 64; ++k) r = r > red[k] ? r : red[k];
        fused_arrive(ws, t, r, G);
      }
      __syncthreads();                                 // red[] is reused by the next tensor's pass 1
    }
    if (t >= 1) {                                      // pass 2 on tensor t-1
      const int tp = t - 1;
      if (threadIdx.x == 0) sh_amax = fused_wait(ws, tp);
      __syncthreads();
      const uint32_t v = sh_amax;
      const float g = v ? __uint_as_float((v & 0x7fffu) << 16) / kGlobalDiv : __builtin_nanf("");
      if (w == 0 && threadIdx.x == 0) gout[tp] = g;
      const double r6 = recip_d6(g);
      build_table(table, g);
      __syncthreads();
      // newest data first: walk the slice's 64-half-block chunks backwards,
      // chunk k going to wave k % 4
      const int64_t off = (int64_t)tp * hb_per_tensor;
      const u32x4* xt = x + off;
      uint32_t* qt = q + off;
      uint8_t* st = sf + off / 2;
      const int64_t nfull = (hi - lo) / 64;              // whole chunks of the slice
      const int nw = kThreads / 64;
      const int wv = wave_id();
      int64_t k = nfull - 1 - wv;
      for (; k - (kU - 1) * nw >= 0; k -= kU * nw) {
        int64_t c[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) c[u] = lo + (k - u * nw) * 64;
        encode_chunks(xt, qt, st, c, r6, table);
      }
      for (; k >= 0; k -= nw) encode_tail(xt, qt, st, lo + k * 64, lo, hi, r6, table);
      if (wv == 0 && lo + nfull * 64 < hi)            // ragged end of the last slice
        encode_tail(xt, qt, st, lo + nfull * 64, lo, hi, r6, table);
      __syncthreads();                                 // the table is rebuilt for the next tensor
    }
  }
  // The last workgroup out restores the header to zero for the next launch.
  // Every counter read of this workgroup has returned (the values were used
  // above), so a relaxed count is enough.
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&((FusedHeader*)ws)->done, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    sh_last = old == (uint32_t)G - 1;
  }
  __syncthreads();
  if (sh_last) {
    const size_t words = (size_t)batch * kTensorWords;
    uint32_t* base = ws + kFusedHeaderBytes / 4;
    for (size_t i = threadIdx.x; i < words; i += kThreads)
      __hip_atomic_store(base + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0)
      __hip_atomic_store(&((FusedHeader*)ws)->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------ fused, tensor held on chip
// When one tensor fits on chip (up to kOnchipMaxPer half blocks per data
// thread, one workgroup per CU), the persistent launch reads every input
// byte from HBM exactly once.
//
// Each workgroup has kOnchipDataWaves data waves and one synchronization
// wave.  Data thread i of workgroup w owns half blocks w*S + p*D + i
// (p < kPer, D data threads, S = D*kPer) of every tensor.  Three tensors are
// on chip at once: t in registers (waiting for its amax, then encoded),
// t+1 in registers (its maximum published, its amax exchange in flight
// while t is encoded) and t+2 streaming into an LDS buffer through direct
// buffer-to-LDS loads, which hold no registers.  A step moves t+1 from LDS
// into registers two pieces at a time, reissuing each freed LDS slot for
// t+2 at once, so HBM always has a tensor's worth of loads queued.
//
// The cross-workgroup exchange of maxima runs in the synchronization wave:
// each workgroup stores its maximum into its own slot of the tensor's line
// set and every synchronization wave polls all slots -- plain agent-scope
// stores and loads, no read-modify-write chains.  Waiting on those loads
// never waits for the data waves' loads (each wave retires its vector
// memory operations through its own in-order counter), and data and
// synchronization waves meet at barriers that order LDS traffic only.
//
// The compiler tracks neither the completion of the buffer-to-LDS loads nor
// reads of what they wrote piecewise, so the data waves wait for them with
// explicit counts: a step always issues the same number of vector memory
// operations in the same order (2*kPer stores, then kPer loads; tensors
// past the batch and slices past a tensor use buffer resources of extent
// zero or of the tensor's size, whose accesses read zeros and write
// nothing).
constexpr int kOnchipDataWaves = 7;
constexpr int kOnchipData = 64 * kOnchipDataWaves;     // data threads per workgroup
constexpr int kOnchipThreads = kOnchipData + 64;      // + the synchronization wave
constexpr int kOnchipMaxPer = 16;                       // 2 x 16 x 16 B registers + 16 x 7 KiB LDS

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with only the vector memory counter constrained (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int kN>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(kN >= 0 && kN < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((kN & 0xF) | ((kN >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier ordering LDS only (the loads and stores in flight stay
// in flight); the memory clobber keeps the compiler's LDS accesses on their
// side of it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Two 16-byte LDS reads, complete on return.
__device__ __forceinline__ void lds_read2(const u32x4* a, const u32x4* b, u32x4& ra, u32x4& rb) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(ra), "=&v"(rb)
               : "v"((uint32_t)(uintptr_t)a), "v"((uint32_t)(uintptr_t)b)
               : "memory");
}

struct OnchipShared {
  double table[128];                  // fp64 reciprocal of every block divisor of the tensor
  double r6;                          // reciprocal of d6 = RN32(6 g)
  uint32_t red[kOnchipDataWaves];     // per-data-wave maxima of the tensor
};

// Buffer resource over tensor t's range of a per-tensor array of `bytes`
// bytes per tensor (t >= batch: extent zero, every access is a no-op).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tensor_rsrc(const void* base, int t, int batch, int64_t bytes) {
  const int tc = t < batch ? t : batch - 1;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)base + (int64_t)tc * bytes), 0,
                                           t < batch ? (int)bytes : 0, kBufferWord3);
}

// Layouts of the on-chip quantize (kMode):
//  kOn1D: the workgroup's slice is S = kPer * D consecutive half blocks;
//      thread i's piece p is half block w S + p D + i (D data threads).
//  kOn2D (16 x 16 tile scales, kPer = 16): thread i of workgroup w owns
//      strip s = w D + i, the 8 columns [8 c, 8 c + 8) of the 16 rows
//      [16 r, 16 r + 16) with (r, c) = (s / spr, s % spr), spr = cols / 8;
//      piece p is row 16 r + p.  Strips 2k and 2k+1 (a lane pair) form one
//      tile; codes and scales are written row-major like the input.
//  kOn2DT (the same tiles, outputs transposed: q [cols][rows/2], sf
//      [cols][rows/16]): data wave v of workgroup w takes the block b = 7 w
//      + v of 8 x 8 strips (128 rows x 64 columns; blocks run down the
//      columns), lane l the strip (8 bR + l / 8, 8 bC + l % 8).  A lane pair
//      is again one tile; for each of its 8 columns a lane writes the 16
//      rows' codes (8 bytes) and the tile's scale byte, so the 8 lanes of a
//      strip column write 64 contiguous bytes of an output row.
// Each lane's input piece p is the 16-byte half block at byte voff + p *
// pstride.  Stores go to qoff + i * qstride and soff + i * sstride, i the
// piece (row-major modes) or the column (kOn2DT).  Lanes past the tensor
// get offsets past its extent: their loads read zeros, their stores are
// dropped.
constexpr int kOn1D = 0, kOn2D = 1, kOn2DT = 2;
constexpr int kOnOutside = 0x70000000;          // past every on-chip tensor's extent, with room for the strides

struct OnchipMap {
  int voff, pstride;                            // input bytes
  int qoff, qstride;                            // code bytes
  int soff, sstride;                            // scale bytes
};

template <int kPer, int kMode>
__device__ __forceinline__ OnchipMap onchip_map(int spr, int srows) {
  OnchipMap m;
  const int lane = (int)threadIdx.x & 63;
  if (kMode == kOn2DT) {
    const int nbr = (srows + 7) / 8, nbc = (spr + 7) / 8;
    const int b = (int)blockIdx.x * kOnchipDataWaves + (int)(threadIdx.x >> 6);
    const int br = b % nbr, bc = b / nbr;
    const int r = 8 * br + (lane >> 3), c = 8 * bc + (lane & 7);
    const bool in = bc < nbc && r < srows && c < spr;
    const int rows = 16 * srows;
    m.voff = in ? (r * 16 * spr + c) * 16 : kOnOutside;
    m.pstride = spr * 16;
    m.qoff = in ? 8 * c * (rows / 2) + 8 * r : kOnOutside;
    m.qstride = rows / 2;
    m.soff = in ? 8 * c * (rows / 16) + r : kOnOutside;
    m.sstride = rows / 16;
    return m;
  }
  if (kMode == kOn2D) {
    const int s = (int)blockIdx.x * kOnchipData + (int)threadIdx.x;
    const int r = s / spr, c = s - r * spr;
    m.voff = (r * 16 * spr + c) * 16;
    m.pstride = spr * 16;
  } else {
    m.voff = ((int)blockIdx.x * kPer * kOnchipData + (int)threadIdx.x) * 16;
    m.pstride = kOnchipData * 16;
  }
  m.qoff = m.voff / 4;
  m.qstride = m.pstride / 4;
  // even lanes write the pair's scale byte; odd lanes aim past the extent
  // (a dropped store), so every lane issues the same stores
  m.soff = (lane & 1) ? (int)0x80000000u : m.voff / 32;
  m.sstride = m.pstride / 32;
  return m;
}

// Issues the buffer-to-LDS loads of pieces [p0, p0 + n) of tensor t.
__device__ __forceinline__ void onchip_dma(u32x4 (*L)[kOnchipData], __amdgpu_buffer_rsrc_t rs, const OnchipMap& mp,
                                           int p0, int n) {
  const int w = threadIdx.x >> 6;
  for (int p = p0; p < p0 + n; ++p)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)&L[p][w * 64], 16, mp.voff, p * mp.pstride, 0, kStreamLoad);
}

template <int kPer>
__device__ __forceinline__ uint32_t onchip_wave_max(const u32x4 (&v)[kPer]) {
  uint32_t m = 0;
#pragma unroll
  for (int p = 0; p < kPer; ++p) m = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m, v[p].x), v[p].y), v[p].z), v[p].w);
  return wave_max_u32(halves_max(m));
}

// Moves tensor t+1 from LDS into nxt and refills the LDS buffer with tensor
// t+2, a pair of pieces at a time.  kStores is the number of vector memory
// operations issued since tensor t+1's loads (the previous step's stores):
// before pair j, the operations younger than its second load are the
// kPer-2-2j later loads of t+1, kStores stores and 2j loads of t+2.
template <int kPer, int kStores>
__device__ __forceinline__ void onchip_refill(const u32x4* __restrict__ x, int t, int batch, int64_t hb,
                                              const OnchipMap& mp, u32x4 (&nxt)[kPer], u32x4 (*L)[kOnchipData]) {
  const __amdgpu_buffer_rsrc_t rs = tensor_rsrc(x, t + 2, batch, hb * 16);
#pragma unroll
  for (int p = 0; p < kPer; p += 2) {
    wait_vmcnt<kPer - 2 + kStores>();
    lds_read2(&L[p][threadIdx.x], &L[p + 1][threadIdx.x], nxt[p], nxt[p + 1]);
    onchip_dma(L, rs, mp, p, 2);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One step of a data wave: tensor t (in cur) is encoded once its amax
// arrives, tensor t+1 moves from LDS into nxt and its maximum is published.
// Vector memory operations the encode of one tensor issues per thread.
template <int kPer, int kMode>
constexpr int onchip_stores() { return kMode == kOn2DT ? 16 : 2 * kPer; }

template <int kPer, int kMode>
__device__ __forceinline__ void onchip_data_step(const u32x4* __restrict__ x, int t, int batch, int64_t hb,
                                                 const OnchipMap& mp, u32x4 (&cur)[kPer], u32x4 (&nxt)[kPer],
                                                 u32x4 (*L)[kOnchipData], uint32_t* __restrict__ q,
                                                 uint8_t* __restrict__ sf, OnchipShared& sh) {
  if (t == 0)
    onchip_refill<kPer, 0>(x, t, batch, hb, mp, nxt, L);
  else
    onchip_refill<kPer, onchip_stores<kPer, kMode>()>(x, t, batch, hb, mp, nxt, L);
  const uint32_t m = onchip_wave_max<kPer>(nxt);
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = m;
  lds_barrier();                                       // maxima of t+1 -> synchronization wave
  lds_barrier();                                       // amax of t, r6 and table <- synchronization wave
  const double r6 = sh.r6;
  const __amdgpu_buffer_rsrc_t rq = tensor_rsrc(q, t, batch, hb * 4);
  const __amdgpu_buffer_rsrc_t rsf = tensor_rsrc(sf, t, batch, hb / 2);
  uint32_t sbyte2d = 0u;
  double rd2d = 0.0;
  if (kMode != kOn1D) {                                // one 16 x 16 tile: the lane's 16 rows and its partner's
    uint32_t bam = 0u;
#pragma unroll
    for (int p = 0; p < kPer; ++p) bam = bam > half_absmax_bits(cur[p]) ? bam : half_absmax_bits(cur[p]);
    sbyte2d = block_scale_byte(pair_max(bam), r6);
    rd2d = sh.table[sbyte2d];
  }
  if (kMode == kOn2DT) {
    // column j of the strip: rows 0..7 and 8..15 gathered into two half
    // blocks (row p in element p), 8 code bytes down the column
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      uint32_t col[8];
#pragma unroll
      for (int p = 0; p < 16; p += 2) {
        const uint32_t lo = j / 2 == 0 ? cur[p].x : j / 2 == 1 ? cur[p].y : j / 2 == 2 ? cur[p].z : cur[p].w;
        const uint32_t hi = j / 2 == 0 ? cur[p + 1].x : j / 2 == 1 ? cur[p + 1].y : j / 2 == 2 ? cur[p + 1].z : cur[p + 1].w;
        col[p / 2] = __builtin_amdgcn_perm(hi, lo, sel);
      }
      const uint32_t c0 = encode_half(u32x4{col[0], col[1], col[2], col[3]}, rd2d);
      const uint32_t c1 = encode_half(u32x4{col[4], col[5], col[6], col[7]}, rd2d);
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{c0, c1}, rq, mp.qoff, j * mp.qstride, 0);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbyte2d, rsf, mp.soff, j * mp.sstride, 0);
      __builtin_amdgcn_sched_barrier(0);               // one column's temporaries at a time
    }
    return;
  }
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    const uint32_t sbyte = kMode == kOn2D ? sbyte2d : block_scale_byte(pair_max(half_absmax_bits(cur[p])), r6);
    const uint32_t code = encode_half(cur[p], kMode == kOn2D ? rd2d : sh.table[sbyte]);
    __builtin_amdgcn_raw_buffer_store_b32(code, rq, mp.qoff, p * mp.qstride, 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbyte, rsf, mp.soff, p * mp.sstride, 0);
    __builtin_amdgcn_sched_barrier(0);                 // one half block's temporaries at a time
  }
}

// Synchronization wave: slot exchange of tensor t's workgroup maxima.
__device__ __forceinline__ void onchip_publish(uint32_t* ws, int t, uint32_t m) {
  __hip_atomic_store(fused_line(ws, t, 0) + blockIdx.x, 0x80000000u | m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls every slot of tensor t until all G are filled; returns the maximum
// (bit 31 set), or 0 after the spin limit (error flag raised).
__device__ __forceinline__ uint32_t onchip_wait(uint32_t* ws, int t, int G) {
  const int lane = threadIdx.x & 63;
  const uint32_t* slots = fused_line(ws, t, 0);
  for (uint32_t it = 0; it < kSpinLimit; ++it) {
    uint32_t mx = 0, ok = 1;
    for (int k = lane; k < G; k += 64) {
      const uint32_t s = __hip_atomic_load(slots + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok &= s >> 31;
      mx = mx > s ? mx : s;
    }
    if (__builtin_amdgcn_ballot_w64(ok == 0) == 0) return wave_max_u32(mx);
    __builtin_amdgcn_s_sleep(1);
  }
  if (lane == 0) __hip_atomic_store(&((FusedHeader*)ws)->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 0u;
}

template <int kPer, int kMode>
__global__ void __launch_bounds__(kOnchipThreads) fused_onchip_kernel(const u32x4* __restrict__ x, int batch,
                                                                      int64_t hb, int spr, int srows, uint32_t* ws,
                                                                      float* __restrict__ gout,
                                                                      uint32_t* __restrict__ q,
                                                                      uint8_t* __restrict__ sf) {
  static_assert(kPer % 2 == 0 && kPer <= kOnchipMaxPer, "pieces move in pairs");
  static_assert(kMode == kOn1D || kPer == 16, "a 2D strip is 16 rows");
  __shared__ OnchipShared sh;
  __shared__ __attribute__((aligned(16))) u32x4 L[kPer][kOnchipData];
  const int G = gridDim.x;
  if (wave_id() < kOnchipDataWaves) {
    u32x4 a[kPer], b[kPer];
    const OnchipMap mp = onchip_map<kPer, kMode>(spr, srows);
    onchip_dma(L, tensor_rsrc(x, 0, batch, hb * 16), mp, 0, kPer);
    wait_vmcnt<0>();
#pragma unroll
    for (int p = 0; p < kPer; p += 2) lds_read2(&L[p][threadIdx.x], &L[p + 1][threadIdx.x], a[p], a[p + 1]);
    onchip_dma(L, tensor_rsrc(x, 1, batch, hb * 16), mp, 0, kPer);
    const uint32_t m = onchip_wave_max<kPer>(a);
    if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = m;
    lds_barrier();                                     // maxima of tensor 0
    int t = 0;
    for (; t + 1 < batch; t += 2) {
      onchip_data_step<kPer, kMode>(x, t, batch, hb, mp, a, b, L, q, sf, sh);
      onchip_data_step<kPer, kMode>(x, t + 1, batch, hb, mp, b, a, L, q, sf, sh);
    }
    if (t < batch) onchip_data_step<kPer, kMode>(x, t, batch, hb, mp, a, b, L, q, sf, sh);
    return;
  }
  // synchronization wave
  const int lane = threadIdx.x & 63;
  auto red_max = [&]() {
    uint32_t r = sh.red[0];
#pragma unroll
    for (int k = 1; k < kOnchipDataWaves; ++k) r = r > sh.red[k] ? r : sh.red[k];
    return r;
  };
  lds_barrier();
  if (lane == 0) onchip_publish(ws, 0, red_max());
  for (int t = 0; t < batch; ++t) {
    lds_barrier();                                     // maxima of t+1 are in sh.red
    const uint32_t next = red_max();
    if (lane == 0 && t + 1 < batch) onchip_publish(ws, t + 1, next);
    const uint32_t v = onchip_wait(ws, t, G);
    const float g = v ? __uint_as_float((v & 0x7fffu) << 16) / kGlobalDiv : __builtin_nanf("");
    sh.table[lane] = recip_entry((uint32_t)lane, g);
    if (lane < 63) sh.table[lane + 64] = recip_entry((uint32_t)lane + 64, g);
    if (lane == 0) {
      sh.r6 = recip_d6(g);
      if (blockIdx.x == 0) gout[t] = g;
    }
    lds_barrier();                                     // publish r6 and the table
  }
  // the last workgroup out restores the slots and the counter to zero; every
  // slot read of this workgroup has returned (the values were used above)
  uint32_t last = 0;
  if (lane == 0)
    last = __hip_atomic_fetch_add(&((FusedHeader*)ws)->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)G - 1;
  if (__builtin_amdgcn_readfirstlane((int)last)) {
    const size_t words = (size_t)batch * kTensorWords;
    uint32_t* base = ws + kFusedHeaderBytes / 4;
    for (size_t i = lane; i < words; i += 64)
      __hip_atomic_store(base + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) __hip_atomic_store(&((FusedHeader*)ws)->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------ dequantize
__global__ void __launch_bounds__(kThreads) dequant_kernel(const uint32_t* __restrict__ q,
                                                           const uint8_t* __restrict__ sf,
                                                           const float* __restrict__ gin, int64_t hb_per_tensor,
                                                           u32x4* __restrict__ y) {
  const int t = blockIdx.y;
  const float g = gin[t];
  const int64_t off = (int64_t)t * hb_per_tensor;
  const uint32_t* qt = q + off;
  const uint8_t* st = sf + off / 2;
  u32x4* yt = y + off;
  const int64_t step = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kU - 1) * step < hb_per_tensor; i += kU * step) {
    uint32_t c[kU];
    uint8_t s[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      c[u] = __builtin_nontemporal_load(qt + i + u * step);
      s[u] = st[(i + u * step) >> 1];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) yt[i + u * step] = dequant_half(c[u], e4m3_value(s[u]), g);
  }
  for (; i < hb_per_tensor; i += step) yt[i] = dequant_half(qt[i], e4m3_value(st[i >> 1]), g);
}

// Clears n words of scratch (the exchange header of a workspace whose
// contents are not guaranteed, before a cooperative launch uses it).
__global__ void __launch_bounds__(kThreads) zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads) p[i] = 0u;
}

}  // namespace nvfp4

// ============================================================ host entry points
namespace {

using namespace nvfp4;

constexpr int kMaxPartials = 2048;

// Workgroups per tensor for a streaming launch: ~16 workgroups per CU in all,
// but at least kU half blocks per lane.
int wgs_per_tensor(int64_t batch, int64_t hb_per_tensor) {
  const int64_t target = (int64_t)nvfp4host::num_cus() * 16;
  int64_t per = (target + batch - 1) / batch;
  const int64_t need = (hb_per_tensor + (int64_t)kThreads * kU - 1) / ((int64_t)kThreads * kU);
  per = std::max<int64_t>(std::min(per, need), 1);
  return (int)std::min<int64_t>(per, 65535);
}

// Workgroups per tensor when every lane takes its kU half blocks once (the
// grid-stride loop only runs past 65535 workgroups).  Workgroups are
// dispatched tensor by tensor, so the stores in flight stay within one or two
// tensors; with ~16 resident workgroups per CU covering all tensors at once,
// the dequantize of 64 x 2048 x 7168 ran 0.49 ms against 0.42 ms.
int one_pass_wgs(int64_t hb_per_tensor) {
  const int64_t need = (hb_per_tensor + (int64_t)kThreads * kU - 1) / ((int64_t)kThreads * kU);
  return (int)std::max<int64_t>(1, std::min<int64_t>(need, 65535));
}

int amax_wgs_per_tensor(int64_t batch, int64_t vec_per_tensor) {
  const int64_t target = (int64_t)nvfp4host::num_cus() * 32;
  int64_t per = (target + batch - 1) / batch;
  const int64_t need = (vec_per_tensor + (int64_t)kThreads * 4 - 1) / ((int64_t)kThreads * 4);
  per = std::min<int64_t>(std::min(per, need), kMaxPartials);
  return (int)std::max<int64_t>(per, 1);
}

nvfp4_status check_shape(int64_t batch, int64_t rows, int64_t cols) {
  if (batch < 0 || rows < 0 || cols < 0 || cols % kBlock) return NVFP4_EINVAL;
  if (batch > 65535) return NVFP4_EINVAL;                        // grid.y
  if (rows > 0 && cols > 0 && rows > (INT64_C(1) << 58) / cols) return NVFP4_EINVAL;
  return NVFP4_OK;
}

size_t fused_header_bytes(int64_t batch) { return kFusedHeaderBytes + (size_t)batch * kTensorWords * 4; }

// Co-resident workgroups for the persistent launch (cached per device).
int fused_grid(int64_t hb_per_tensor) {
  static int per_cu = -1;
  if (per_cu < 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fused_quantize_kernel, kThreads, 0) != hipSuccess || nb < 1)
      nb = 1;
    per_cu = std::min(nb, 4);
  }
  int64_t g = (int64_t)nvfp4host::num_cus() * per_cu;
  const int64_t need = std::max<int64_t>(1, (hb_per_tensor + 255) / 256);
  return (int)std::max<int64_t>(1, std::min(g, need));
}

// Half blocks per data thread for the on-chip persistent launch: the
// smallest even count that covers a tensor with at most one workgroup per
// CU, or 0 when the tensor is too large to hold on chip (the streaming
// launch runs then).
int onchip_per_thread(int64_t hb_per_tensor) {
  if (hb_per_tensor <= 0) return 0;
  const int64_t cus = nvfp4host::num_cus();
  if (cus > (int64_t)kTensorWords) return 0;           // one exchange slot per workgroup
  const int64_t cap = cus * kOnchipData;
  int64_t per = (hb_per_tensor + cap - 1) / cap;
  per += per & 1;                                       // pieces move in pairs
  return per <= kOnchipMaxPer ? (int)per : 0;
}

}  // namespace

namespace nvfp4host {

// Scratch bytes of quantize_2d_onchip for a batch (the exchange header).
size_t quantize_2d_onchip_ws_bytes(int64_t batch) {
  return batch <= 0 ? 0 : (fused_header_bytes(batch) + 255) & ~(size_t)255;
}

// 2D quantize (one E4M3 scale per 16 x 16 tile; outputs row-major, or
// transposed with colwise) of batch tensors [rows][cols] in one cooperative
// launch of fused_onchip_kernel<16, kOn2D | kOn2DT> when a tensor's 16-row x
// 8-column strips fit on the chip: every input byte is read once.  ENOTSUP when they do not (the
// caller then runs its two-pass path).  The exchange header in ws is
// cleared first, so the scratch needs no preparation.  The shape and
// pointers are validated by the caller (rows % 16 == 0, cols % 16 == 0).
nvfp4_status quantize_2d_onchip(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, bool colwise, uint8_t* q,
                                uint8_t* sf, float* g, void* ws, hipStream_t s) {
  if (batch <= 0 || rows <= 0 || cols <= 0) return NVFP4_ENOTSUP;
  const int64_t cus = num_cus();
  if (cus > (int64_t)kTensorWords) return NVFP4_ENOTSUP;   // one exchange slot per workgroup
  const int64_t srows = rows / 16, spr = cols / 8;
  const int64_t G = colwise ? (((srows + 7) / 8) * ((spr + 7) / 8) + kOnchipDataWaves - 1) / kOnchipDataWaves
                            : (srows * spr + kOnchipData - 1) / kOnchipData;
  if (G > cus) return NVFP4_ENOTSUP;
  const int64_t words = (int64_t)(quantize_2d_onchip_ws_bytes(batch) / 4);
  zero_words_kernel<<<(unsigned)std::min<int64_t>((words + kThreads - 1) / kThreads, 1024), kThreads, 0, s>>>(
      (uint32_t*)ws, words);
  NVFP4_LAUNCH_CHECK();
  const u32x4* xa = (const u32x4*)x;
  int bt = (int)batch;
  int64_t hb = rows * cols / 8;
  int spri = (int)spr, srowsi = (int)srows;       // a tensor that fits on chip has far fewer than 2^31 of either
  uint32_t* wsa = (uint32_t*)ws;
  uint32_t* qa = (uint32_t*)q;
  void* args[] = {&xa, &bt, (void*)&hb, &spri, &srowsi, &wsa, &g, &qa, &sf};
  const void* fn = colwise ? (const void*)fused_onchip_kernel<16, kOn2DT> : (const void*)fused_onchip_kernel<16, kOn2D>;
  const hipError_t e = hipLaunchCooperativeKernel(fn, dim3((unsigned)G), dim3(kOnchipThreads), args, 0, s);
  if (e != hipSuccess) {
    set_hip_error(e);
    return NVFP4_EHIP;
  }
  return NVFP4_OK;
}

}  // namespace nvfp4host

extern "C" {

size_t nvfp4_quantize_workspace_bytes(int64_t batch, int64_t rows, int64_t cols) {
  if (batch <= 0 || rows < 0 || cols < 0) return 0;
  (void)rows;
  (void)cols;
  // fused header, then the two-kernel path's per-tensor partial maxima
  const size_t head = (fused_header_bytes(batch) + 255) & ~(size_t)255;
  return head + (size_t)batch * kMaxPartials * sizeof(uint32_t);
}

nvfp4_status nvfp4_quantize(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sf,
                            float* g, void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  nvfp4_status st = check_shape(batch, rows, cols);
  if (st) return st;
  if (flags != NVFP4_TWO_KERNEL && flags != NVFP4_FUSED) return NVFP4_ENOTSUP;
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
  const int64_t hb = n / 8;
  if (flags == NVFP4_FUSED) {
    const int onchip_per = onchip_per_thread(hb);
    if (onchip_per > 0) {
      const u32x4* xa = (const u32x4*)x;
      int bt = (int)batch;
      uint32_t* ws = (uint32_t*)workspace;
      uint32_t* qa = (uint32_t*)q;
      int spr = 0, srows = 0;                          // unused by the 1D layout
      void* args[] = {&xa, &bt, (void*)&hb, &spr, &srows, &ws, &g, &qa, &sf};
      const int64_t slice = (int64_t)onchip_per * kOnchipData;
      const int G = (int)((hb + slice - 1) / slice);
      const void* fn = nullptr;
      const void* fns[kOnchipMaxPer / 2] = {
          (const void*)fused_onchip_kernel<2, kOn1D>,
          (const void*)fused_onchip_kernel<4, kOn1D>,
          (const void*)fused_onchip_kernel<6, kOn1D>,
          (const void*)fused_onchip_kernel<8, kOn1D>,
          (const void*)fused_onchip_kernel<10, kOn1D>,
          (const void*)fused_onchip_kernel<12, kOn1D>,
          (const void*)fused_onchip_kernel<14, kOn1D>,
          (const void*)fused_onchip_kernel<16, kOn1D>,
      };
      fn = fns[onchip_per / 2 - 1];
      hipError_t e = hipLaunchCooperativeKernel(fn, dim3(G), dim3(kOnchipThreads), args, 0, s);
      if (e != hipSuccess) {
        nvfp4host::set_hip_error(e);
        return NVFP4_EHIP;
      }
      return NVFP4_OK;
    }
    const int G = fused_grid(hb);
    const u32x4* xa = (const u32x4*)x;
    int bt = (int)batch;
    uint32_t* ws = (uint32_t*)workspace;
    uint32_t* qa = (uint32_t*)q;
    void* args[] = {&xa, &bt, (void*)&hb, &ws, &g, &qa, &sf};
    hipError_t e = hipLaunchCooperativeKernel((const void*)fused_quantize_kernel, dim3(G), dim3(kThreads), args, 0, s);
    if (e != hipSuccess) {
      nvfp4host::set_hip_error(e);
      return NVFP4_EHIP;
    }
    return NVFP4_OK;
  }
  const size_t head = (fused_header_bytes(batch) + 255) & ~(size_t)255;
  uint32_t* partial = (uint32_t*)((char*)workspace + head);
  const int64_t vec = hb;
  const int p1 = amax_wgs_per_tensor(batch, vec);
  amax_partial_kernel<<<dim3(p1, (unsigned)batch), kThreads, 0, s>>>((const u32x4*)x, vec, partial);
  NVFP4_LAUNCH_CHECK();
  const int p2 = wgs_per_tensor(batch, hb);
  encode_kernel<true><<<dim3(p2, (unsigned)batch), kThreads, 0, s>>>((const u32x4*)x, hb, partial, p1, nullptr, g,
                                                                      (uint32_t*)q, sf);
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
  const int64_t hb = n / 8;
  const int p2 = wgs_per_tensor(batch, hb);
  encode_kernel<false><<<dim3(p2, (unsigned)batch), kThreads, 0, s>>>((const u32x4*)x, hb, nullptr, 0, g, nullptr,
                                                                       (uint32_t*)q, sf);
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
  const int64_t hb = n / 8;
  const int p = one_pass_wgs(hb);
  dequant_kernel<<<dim3(p, (unsigned)batch), kThreads, 0, s>>>((const uint32_t*)q, sf, g, hb, (u32x4*)y);
  NVFP4_LAUNCH_CHECK();
  return NVFP4_OK;
}

}  // extern "C"
