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
//  FUSED       one launch of co-resident workgroups that walk the batch
//              tensor by tensor.  fused_reg8_kernel when a tensor fits on
//              chip (registers + LDS of the whole GPU): every input byte is
//              read from HBM once.  fused_big_kernel for a larger tensor:
//              up to four chunks stay on chip between its two passes.
//              Past 2 GiB per tensor, fused_quantize_kernel: each workgroup
//              reduces its slice of tensor t, publishes it (agent-scope
//              atomics), then encodes its slice of tensor t-1, read again
//              newest-first.
// The 2D tile-scale variants (nvfp4_quantize_ex) run fused_2d_reg_kernel
// when the tensors fit on chip.
#include <algorithm>
#include <atomic>
#include <cstddef>
#include <utility>

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
// Polls of a bounded wait before it gives up (~seconds at the default: only
// a grid that is not fully resident gets there).  Per device; set by
// nvfp4_set_wait_limit, read by every wait of the co-resident kernels.
constexpr uint32_t kDefaultWaitLimit = 1u << 24;
__device__ uint32_t g_wait_limit = kDefaultWaitLimit;

// done counts the workgroups out of a launch (the last one restores the
// exchange words to zero); error is set by any wait that gave up and stays
// set until nvfp4_quantize_status reads and clears it.
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
  const uint32_t limit = g_wait_limit;
  for (uint32_t it = 0; it < limit; ++it) {
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

// ------------------------------------------------------------ on-chip pipeline helpers
// The on-chip kernels below hold whole tensors in registers and LDS (one
// workgroup per CU) and exchange per-tensor maxima between workgroups
// through one slot per workgroup in the workspace: plain agent-scope stores
// and polled loads, no read-modify-write chains.  A wave retires its vector
// memory operations through one in-order counter, and the compiler tracks
// neither buffer-to-LDS loads nor reads of what they wrote piecewise, so the
// kernels issue the same memory operations in the same order in every wave
// and wait with explicit counts.
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

// Buffer resource over tensor t's range of a per-tensor array of `bytes`
// bytes per tensor (t >= batch: extent zero, every access is a no-op).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tensor_rsrc(const void* base, int t, int batch, int64_t bytes) {
  const int tc = t < batch ? t : batch - 1;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)base + (int64_t)tc * bytes), 0,
                                           t < batch ? (int)bytes : 0, kBufferWord3);
}

constexpr int kOnOutside = 0x70000000;          // past every on-chip tensor's extent, with room for the strides

// Slot exchange: workgroup w publishes its maximum of tensor t.
__device__ __forceinline__ void onchip_publish(uint32_t* ws, int t, uint32_t m) {
  __hip_atomic_store(fused_line(ws, t, 0) + blockIdx.x, 0x80000000u | m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls every slot of tensor t until all G are filled; returns the maximum
// (bit 31 set), or 0 after the spin limit (error flag raised).
__device__ __forceinline__ uint32_t onchip_wait(uint32_t* ws, int t, int G) {
  const int lane = threadIdx.x & 63;
  // One 16-byte load per lane reads 256 slots (a few cache lines per poll
  // instead of a request per slot).  The loads carry the agent-coherent
  // cache policy of a relaxed agent-scope atomic load (sc1), and each slot
  // is one aligned word written by one atomic store, so no slot tears.  The
  // resource spans the tensor's line set: words past it read as zero and
  // words past G count as filled.
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(fused_line(ws, t, 0), 0, (int)(kTensorWords * 4), kBufferWord3);
  const uint32_t limit = g_wait_limit;
  for (uint32_t it = 0; it < limit; ++it) {
    uint32_t mx = 0, ok = 1;
    for (int base = 0; base < G; base += 256) {
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (base + 4 * lane) * 4, 0,
                                                                                      kCoherentLoad));
      const int i = base + 4 * lane;
      ok &= (i >= G || (v.x >> 31)) && (i + 1 >= G || (v.y >> 31)) && (i + 2 >= G || (v.z >> 31)) &&
            (i + 3 >= G || (v.w >> 31));
      const uint32_t m2 = v.x > v.y ? v.x : v.y, m3 = v.z > v.w ? v.z : v.w;
      const uint32_t m4 = m2 > m3 ? m2 : m3;
      mx = mx > m4 ? mx : m4;
    }
    if (__builtin_amdgcn_ballot_w64(ok == 0) == 0) return wave_max_u32(mx);
    __builtin_amdgcn_s_sleep(4);
  }
  if (lane == 0) __hip_atomic_store(&((FusedHeader*)ws)->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 0u;
}

// One LDS read of 16 bytes at base + kOff (an immediate offset), complete on
// return.
template <int kOff>
__device__ __forceinline__ u32x4 lds_read_at(uint32_t base) {
  static_assert(kOff >= 0 && kOff < 65536, "ds_read offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2\n\ts_waitcnt lgkmcnt(0)" : "=v"(r) : "v"(base), "i"(kOff) : "memory");
  return r;
}

// Block maxima kept beside a register set: the pair maximum (bf16 magnitude
// bits of the 16-value block) of piece p in half p & 1 of word p / 2.
template <int kPer>
struct BlockMax {
  uint32_t w[kPer / 2];
};

template <int kPer>
__device__ __forceinline__ uint32_t bm_get(const BlockMax<kPer>& bm, int p) {
  return (p & 1) ? bm.w[p / 2] >> 16 : bm.w[p / 2] & 0xffffu;
}
// bam << 16 as a float: the block amax (the halves' other bits are zero).
template <int kPer>
__device__ __forceinline__ float bm_value(const BlockMax<kPer>& bm, int p) {
  return __uint_as_float((p & 1) ? bm.w[p / 2] & 0xffff0000u : bm.w[p / 2] << 16);
}
template <int kPer>
__device__ __forceinline__ void bm_set(BlockMax<kPer>& bm, int p, uint32_t h) {
  bm.w[p / 2] = (p & 1) ? __builtin_amdgcn_perm(h, bm.w[p / 2], 0x05040100u)    // h into the high half
                        : __builtin_amdgcn_perm(h, bm.w[p / 2], 0x03020504u);   // h into the low half
}

// Block maxima of a whole set (prologue); returns the wave maximum.
template <int kPer>
__device__ __forceinline__ uint32_t set_block_max(const u32x4 (&R)[kPer], BlockMax<kPer>& bm) {
  uint32_t m = 0;
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    const uint32_t h = pair_max(half_absmax_bits(R[p]));
    m = m > h ? m : h;
    if (p & 1) bm.w[p / 2] |= h << 16;
    else bm.w[p / 2] = h;
  }
  return wave_max_u32(m);
}

// ------------------------------------------------------------ fused, four tensors on chip
// The 1D FUSED quantize when one tensor fits on chip.  Data thread i (of
// D = 512) of workgroup w owns half blocks w*S + p*D + i (p < kPer, S =
// kPer*D) of every tensor, so every load and store instruction of a wave is
// one contiguous run.  Four tensors are on chip at once: three in register
// sets and one in an LDS stage.  Step t, piece by piece: encode piece p of
// tensor t (its set) and store its codes and scale byte; move the stage's
// piece p (tensor t+3) into the freed registers, taking its block maximum;
// reload that stage slot with tensor t+4 by a buffer-to-LDS load (which
// holds no registers).  The encode (VALU), the move (LDS) and the memory
// operations of a wave interleave, and the eight waves (two per SIMD)
// overlap them.
//
// A tensor's maximum is taken when it enters registers, three steps before
// its encode.  Wave 7 does the exchange:
//   - at the start of step t it publishes the workgroup's maximum of t+2
//     (one agent-scope store into the workgroup's slot);
//   - also at the start of step t it polls the slots of t+1 with a
//     buffer-to-LDS load (so it never waits on the poll while its data loads
//     are in flight), checks them at the end of step t and builds t+1's
//     table of reciprocals before the step's single barrier.  Only if some
//     workgroup has not published yet does it fall back to a bounded wait.
// So each maximum is published a step before anyone polls it and two steps
// before anyone needs it: a slow workgroup (late data, a slow fabric round
// trip) holds up the others only when it falls that far behind.
//
// The compiler does not track buffer-to-LDS loads, so the waits are
// explicit.  Every wave issues the same memory operations in the same order
// (the other waves aim the exchange's store and two loads at zero-extent
// resources), so the counts are the same constants in every wave: the stage
// load of piece p issued a step earlier has 3*kPer + 2 younger operations
// when piece p is moved, and the poll load 3*kPer at the end of the step.
// Steps run in groups of three (the register sets rotate), then one or two
// steps finish a batch that is not a multiple of three.
constexpr int kR8Waves = 8;
constexpr int kR8Data = 64 * kR8Waves;                 // data threads per workgroup
constexpr int kR8MaxPer = 14;                          // 3 sets x 14 x 16 B in registers + 14 x 8 KiB of LDS
constexpr int kR8StagePiece = kR8Data * 16;            // 8192 bytes per stage piece
constexpr int kR8StageSplit = 65536 / kR8StagePiece;   // pieces reachable from the first base (8)
constexpr int kR8PollSlots = 512;                      // slots one step's two poll loads cover

struct Reg8Shared {
  double table[2][128];               // fp64 reciprocal of every block divisor, tensors of either parity
  double r6[2];                       // reciprocal of d6 = RN32(6 g)
  uint32_t red[2][kR8Waves];          // per-wave maxima of t+3, by the parity of the step t
  uint32_t red0[3][kR8Waves];         // per-wave maxima of tensors 0..2 (prologue)
  u32x4 poll[kR8Waves][2][64];        // each wave's poll landing area (only wave 7's is read)
};

template <int kPer, int p>
__device__ __forceinline__ u32x4 r8_stage_read(uint32_t b0, uint32_t b1) {
  if constexpr (p < kR8StageSplit) return lds_read_at<p * kR8StagePiece>(b0);
  else return lds_read_at<(p - kR8StageSplit) * kR8StagePiece>(b1);
}

template <int kPer, int p, int kWait>
__device__ __forceinline__ void r8_piece(u32x4 (&cur)[kPer], BlockMax<kPer>& bm, uint32_t& m, double r6,
                                         const double* table, __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rsf,
                                         __amdgpu_buffer_rsrc_t rx, int qoff, int soff, int voff, uint32_t b0,
                                         uint32_t b1, lds_void_t* stage_w) {
  const uint32_t sbyte = e4m3_rne_sat(rn32((double)bm_value<kPer>(bm, p) * r6));
  const uint32_t code = encode_half(cur[p], table[sbyte]);
  // codes stream out non-temporal (whole lines: 0.431 -> 0.426 ms on the
  // experts, alternating with the dequantize); the scale bytes, 32-byte runs
  // per store, go through L2, which merges them into lines (0.410 -> 0.401
  // ms for the quantize and 0.393 -> 0.385 ms for the dequantize after it,
  // which reads them back)
  __builtin_amdgcn_raw_buffer_store_b32(code, rq, qoff, p * kR8Data * 4, kStreamLoad);
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbyte, rsf, soff, p * (kR8Data / 2), 0);
  wait_vmcnt<kWait>();                                 // stage piece p (issued a step earlier) has landed
  cur[p] = r8_stage_read<kPer, p>(b0, b1);
  const uint32_t h = pair_max(half_absmax_bits(cur[p]));
  m = m > h ? m : h;
  bm_set<kPer>(bm, p, h);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)((__attribute__((address_space(3))) char*)stage_w +
                                                             p * kR8StagePiece),
                                           16, voff, p * kR8StagePiece, 0, kStreamLoad);
  __builtin_amdgcn_sched_barrier(0);                   // keep each piece's operations in this order
}

template <int kPer, int kWait, int... P>
__device__ __forceinline__ void r8_pieces(std::integer_sequence<int, P...>, u32x4 (&cur)[kPer], BlockMax<kPer>& bm,
                                          uint32_t& m, double r6, const double* table, __amdgpu_buffer_rsrc_t rq,
                                          __amdgpu_buffer_rsrc_t rsf, __amdgpu_buffer_rsrc_t rx, int qoff, int soff,
                                          int voff, uint32_t b0, uint32_t b1, lds_void_t* stage_w) {
  (r8_piece<kPer, P, kWait>(cur, bm, m, r6, table, rq, rsf, rx, qoff, soff, voff, b0, b1, stage_w), ...);
}

// Table of tensor t from its amax (bit 31 set), or NaN after a wait gave up.
__device__ __forceinline__ void r8_table(Reg8Shared& sh, int t, uint32_t v, float* __restrict__ gout) {
  const int lane = threadIdx.x & 63;
  const float g = v ? __uint_as_float((v & 0x7fffu) << 16) / kGlobalDiv : __builtin_nanf("");
  sh.table[t & 1][lane] = recip_entry((uint32_t)lane, g);
  if (lane < 63) sh.table[t & 1][lane + 64] = recip_entry((uint32_t)lane + 64, g);
  if (lane == 0) {
    sh.r6[t & 1] = recip_d6(g);
    if (blockIdx.x == 0) gout[t] = g;
  }
}

__device__ __forceinline__ uint32_t r8_red_max(const uint32_t* red) {
  uint32_t r = red[0];
#pragma unroll
  for (int k = 1; k < kR8Waves; ++k) r = r > red[k] ? r : red[k];
  return r;
}

// The three memory operations that open a step: wave 7 publishes (when
// there is a maximum to publish) and polls tensor tp's slots; every other
// wave, and wave 7 when there is nothing to do, aims them at zero-extent
// resources.
__device__ __forceinline__ void r8_exchange_ops(uint32_t* ws, int G, int tpub, uint32_t mpub, int tp, bool do_poll,
                                                Reg8Shared& sh) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const bool mine = wave == kR8Waves - 1;
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(ws, 0, 0, kBufferWord3);
  if (mine && tpub >= 0) {
    if (lane == 0) onchip_publish(ws, tpub, mpub);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(0u, none, 0, 0, 0);
  }
  const int ext = (mine && do_poll) ? G * 4 : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(fused_line(ws, tp < 0 ? 0 : tp, 0), 0, ext,
                                                                      kBufferWord3);
  lds_void_t* dst = (lds_void_t*)(uintptr_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)&sh.poll[wave][0][0]);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, lane * 16, 0, 0, kCoherentLoad);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)((__attribute__((address_space(3))) char*)dst + 1024), 16,
                                           lane * 16, 1024, 0, kCoherentLoad);
  __builtin_amdgcn_sched_barrier(0);
}

// Wave 7 at the end of step t: the polled slots of tensor tp (landed: the
// step's wait covers them), or a bounded wait if some workgroup is behind.
__device__ __forceinline__ uint32_t r8_gather(uint32_t* ws, int tp, int G, const Reg8Shared& sh) {
  const int lane = threadIdx.x & 63;
  uint32_t mx = 0, ok = 1;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 v = sh.poll[kR8Waves - 1][h][lane];
    const int i = h * 256 + 4 * lane;
    ok &= (i >= G || (v.x >> 31)) && (i + 1 >= G || (v.y >> 31)) && (i + 2 >= G || (v.z >> 31)) &&
          (i + 3 >= G || (v.w >> 31));
    const uint32_t m2 = v.x > v.y ? v.x : v.y, m3 = v.z > v.w ? v.z : v.w;
    const uint32_t m4 = m2 > m3 ? m2 : m3;
    mx = mx > m4 ? mx : m4;
  }
  if (__builtin_amdgcn_ballot_w64(ok == 0) == 0) return wave_max_u32(mx);
  return onchip_wait(ws, tp, G);
}

template <int kPer>
__device__ __forceinline__ void r8_step(const u32x4* __restrict__ x, int t, int batch, int64_t hb, int voff, int qoff,
                                        int soff, u32x4 (&cur)[kPer], BlockMax<kPer>& bm, uint32_t b0, uint32_t b1,
                                        lds_void_t* stage_w, uint32_t* ws, int G, float* __restrict__ gout,
                                        uint32_t* __restrict__ q, uint8_t* __restrict__ sf, Reg8Shared& sh) {
  lds_barrier();                                       // t's table is ready; the maxima of t+2 were reduced
  const bool pub = t >= 1 && t + 2 < batch;
  r8_exchange_ops(ws, G, pub ? t + 2 : -1, pub ? r8_red_max(sh.red[(t - 1) & 1]) : 0u, t + 1, t + 1 < batch, sh);
  const double r6 = sh.r6[t & 1];
  const double* table = sh.table[t & 1];
  const __amdgpu_buffer_rsrc_t rq = tensor_rsrc(q, t, batch, hb * 4);
  const __amdgpu_buffer_rsrc_t rsf = tensor_rsrc(sf, t, batch, hb / 2);
  const __amdgpu_buffer_rsrc_t rx = tensor_rsrc(x, t + 4, batch, hb * 16);   // extent zero past the batch
  uint32_t m = 0;
  r8_pieces<kPer, 3 * kPer + 2>(std::make_integer_sequence<int, kPer>{}, cur, bm, m, r6, table, rq, rsf, rx, qoff, soff,
                                voff, b0,
                  b1, stage_w);
  sh.red[t & 1][wave_id()] = wave_max_u32(m);          // wave-uniform value and address
  wait_vmcnt<3 * kPer>();                              // the poll loads of this step have landed
  if (wave_id() == kR8Waves - 1 && t + 1 < batch) r8_table(sh, t + 1, r8_gather(ws, t + 1, G, sh), gout);
}

template <int kPer>
__global__ void __launch_bounds__(kR8Data) fused_reg8_kernel(const u32x4* __restrict__ x, int batch, int64_t hb,
                                                             uint32_t* ws, float* __restrict__ gout,
                                                             uint32_t* __restrict__ q, uint8_t* __restrict__ sf) {
  static_assert(kPer % 2 == 0 && kPer <= kR8MaxPer, "pieces in pairs, within the register budget");
  __shared__ Reg8Shared sh;
  __shared__ __attribute__((aligned(16))) u32x4 L[kPer][kR8Data];
  const int G = gridDim.x;
  const int lane = (int)threadIdx.x & 63, wave = wave_id();
  const int voff = ((int)blockIdx.x * kPer * kR8Data + (int)threadIdx.x) * 16;
  const int qoff = voff / 4;
  // even lanes write the pair's scale byte; odd lanes aim past the extent
  const int soff = (lane & 1) ? (int)0x80000000u : voff / 32;
  u32x4 a[kPer], b[kPer], c[kPer];
  BlockMax<kPer> am, bmx, cm;
  {
    const __amdgpu_buffer_rsrc_t r0 = tensor_rsrc(x, 0, batch, hb * 16), r1 = tensor_rsrc(x, 1, batch, hb * 16),
                                 r2 = tensor_rsrc(x, 2, batch, hb * 16);
#pragma unroll
    for (int p = 0; p < kPer; ++p)
      a[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r0, voff, p * kR8StagePiece, kStreamLoad));
#pragma unroll
    for (int p = 0; p < kPer; ++p)
      b[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, voff, p * kR8StagePiece, kStreamLoad));
#pragma unroll
    for (int p = 0; p < kPer; ++p)
      c[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r2, voff, p * kR8StagePiece, kStreamLoad));
    __builtin_amdgcn_sched_barrier(0);
  }
  const uint32_t b0 = (uint32_t)(uintptr_t)&L[0][threadIdx.x];
  const uint32_t b1 = b0 + kR8StageSplit * kR8StagePiece;
  lds_void_t* const stage_w =
      (lds_void_t*)(uintptr_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)&L[0][threadIdx.x & ~63]);
  {
    // tensor 3 into the stage, each piece after two stores aimed at
    // zero-extent resources: the memory operations of a step, in order
    const __amdgpu_buffer_rsrc_t nq = tensor_rsrc(q, batch, batch, 0), ns = tensor_rsrc(sf, batch, batch, 0);
    const __amdgpu_buffer_rsrc_t rx = tensor_rsrc(x, 3, batch, hb * 16);
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      __builtin_amdgcn_raw_buffer_store_b32(0u, nq, qoff, p * kR8Data * 4, 0);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)0, ns, soff, p * (kR8Data / 2), 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_void_t*)((__attribute__((address_space(3))) char*)stage_w + p * kR8StagePiece), 16, voff,
          p * kR8StagePiece, 0, kStreamLoad);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  sh.red0[0][wave] = set_block_max<kPer>(a, am);
  sh.red0[1][wave] = set_block_max<kPer>(b, bmx);
  sh.red0[2][wave] = set_block_max<kPer>(c, cm);
  lds_barrier();                                       // maxima of tensors 0..2
  if (wave == kR8Waves - 1) {
    if (lane == 0)
      for (int k = 0; k < 3 && k < batch; ++k) onchip_publish(ws, k, r8_red_max(sh.red0[k]));
    r8_table(sh, 0, onchip_wait(ws, 0, G), gout);
  }
  int t = 0;
  for (; t + 3 <= batch; t += 3) {
    r8_step<kPer>(x, t, batch, hb, voff, qoff, soff, a, am, b0, b1, stage_w, ws, G, gout, q, sf, sh);
    r8_step<kPer>(x, t + 1, batch, hb, voff, qoff, soff, b, bmx, b0, b1, stage_w, ws, G, gout, q, sf, sh);
    r8_step<kPer>(x, t + 2, batch, hb, voff, qoff, soff, c, cm, b0, b1, stage_w, ws, G, gout, q, sf, sh);
  }
  if (t < batch) r8_step<kPer>(x, t, batch, hb, voff, qoff, soff, a, am, b0, b1, stage_w, ws, G, gout, q, sf, sh);
  if (t + 1 < batch) r8_step<kPer>(x, t + 1, batch, hb, voff, qoff, soff, b, bmx, b0, b1, stage_w, ws, G, gout, q, sf, sh);
  wait_vmcnt<0>();                                     // no stage or poll load still writing LDS at exit
  if (wave != kR8Waves - 1) return;
  // the last workgroup out restores the slots and the counter to zero; every
  // slot store of this workgroup has completed (the wait above)
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

// ------------------------------------------------------------ fused 2D scales, four tensors on chip
// The 16 x 16 tile-scale quantize (2D weights) on the same pipeline as
// fused_reg8_kernel: three register sets, one LDS stage, eight waves, the
// exchange in wave 7 a step ahead.  Data thread i of workgroup w owns strip
// s = 512 w + i: the 8 columns [8 c, 8 c + 8) of the 16 rows [16 r, 16 r +
// 16), (r, c) = (s / spr, s % spr), spr = cols / 8; piece p is row 16 r + p,
// so consecutive threads read consecutive 16-byte runs of a row.  Strips 2k
// and 2k+1 (a lane pair) form one tile: its amax is the pair's maximum over
// all 16 pieces, taken when the tensor enters registers, and one scale byte
// and one reciprocal serve every piece of the step.  Codes and scale bytes
// go out row-major like the input (every row of the tile carries the
// tile's byte).  The memory operations of a step, and so the waits, are
// those of the 1D kernel.
constexpr int kR2Per = 16;                             // rows of a strip

template <int p, int kWait>
__device__ __forceinline__ void r2_piece(u32x4 (&cur)[kR2Per], uint32_t& m, double rd, uint32_t sbyte,
                                         __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rsf,
                                         __amdgpu_buffer_rsrc_t rx, int qoff, int soff, int voff, int qstride,
                                         int sstride, int pstride, uint32_t b0, uint32_t b1, lds_void_t* stage_w) {
  const uint32_t code = encode_half(cur[p], rd);
  __builtin_amdgcn_raw_buffer_store_b32(code, rq, qoff, p * qstride, kStreamLoad);
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbyte, rsf, soff, p * sstride, 0);
  wait_vmcnt<kWait>();                                 // stage piece p (issued a step earlier) has landed
  cur[p] = r8_stage_read<kR2Per, p>(b0, b1);
  const uint32_t h = half_absmax_bits(cur[p]);
  m = m > h ? m : h;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)((__attribute__((address_space(3))) char*)stage_w +
                                                             p * kR8StagePiece),
                                           16, voff, p * pstride, 0, kStreamLoad);
  __builtin_amdgcn_sched_barrier(0);                   // keep each piece's operations in this order
}

template <int kWait, int... P>
__device__ __forceinline__ void r2_pieces(std::integer_sequence<int, P...>, u32x4 (&cur)[kR2Per], uint32_t& m,
                                          double rd, uint32_t sbyte, __amdgpu_buffer_rsrc_t rq,
                                          __amdgpu_buffer_rsrc_t rsf, __amdgpu_buffer_rsrc_t rx, int qoff, int soff,
                                          int voff, int qstride, int sstride, int pstride, uint32_t b0, uint32_t b1,
                                          lds_void_t* stage_w) {
  (r2_piece<P, kWait>(cur, m, rd, sbyte, rq, rsf, rx, qoff, soff, voff, qstride, sstride, pstride, b0, b1, stage_w),
   ...);
}

// Tile maximum of a register set (the pair's maximum over its pieces);
// returns the wave maximum.
__device__ __forceinline__ uint32_t set_tile_max(const u32x4 (&R)[kR2Per], uint32_t& tile) {
  uint32_t m = 0;
#pragma unroll
  for (int p = 0; p < kR2Per; ++p) {
    const uint32_t h = half_absmax_bits(R[p]);
    m = m > h ? m : h;
  }
  tile = pair_max(m);
  return wave_max_u32(m);
}

__device__ __forceinline__ void r2_step(const u32x4* __restrict__ x, int t, int batch, int64_t hb, int voff, int qoff,
                                        int soff, int qstride, int sstride, int pstride, u32x4 (&cur)[kR2Per],
                                        uint32_t& tile, uint32_t b0, uint32_t b1, lds_void_t* stage_w, uint32_t* ws,
                                        int G, float* __restrict__ gout, uint32_t* __restrict__ q,
                                        uint8_t* __restrict__ sf, Reg8Shared& sh) {
  lds_barrier();                                       // t's table is ready; the maxima of t+2 were reduced
  const bool pub = t >= 1 && t + 2 < batch;
  r8_exchange_ops(ws, G, pub ? t + 2 : -1, pub ? r8_red_max(sh.red[(t - 1) & 1]) : 0u, t + 1, t + 1 < batch, sh);
  const double r6 = sh.r6[t & 1];
  const uint32_t sbyte = block_scale_byte(tile, r6);
  const double rd = sh.table[t & 1][sbyte];
  const __amdgpu_buffer_rsrc_t rq = tensor_rsrc(q, t, batch, hb * 4);
  const __amdgpu_buffer_rsrc_t rsf = tensor_rsrc(sf, t, batch, hb / 2);
  const __amdgpu_buffer_rsrc_t rx = tensor_rsrc(x, t + 4, batch, hb * 16);   // extent zero past the batch
  uint32_t m = 0;
  r2_pieces<3 * kR2Per + 2>(std::make_integer_sequence<int, kR2Per>{}, cur, m, rd, sbyte, rq, rsf, rx, qoff, soff, voff,
                            qstride, sstride, pstride, b0, b1, stage_w);
  tile = pair_max(m);                                  // tensor t+3, now in this set
  sh.red[t & 1][wave_id()] = wave_max_u32(m);          // wave-uniform value and address
  wait_vmcnt<3 * kR2Per>();                            // the poll loads of this step have landed
  if (wave_id() == kR8Waves - 1 && t + 1 < batch) r8_table(sh, t + 1, r8_gather(ws, t + 1, G, sh), gout);
}

// The COLWISE step (outputs transposed: q [cols][rows/2], sf [cols][rows/16]):
// a column's 16 rows come from all 16 pieces, so the step first encodes the
// strip's 8 columns (two half blocks each, gathered with byte permutes; 8
// code bytes and the tile's byte per column, the 8 lanes of a strip column
// writing 64 contiguous bytes of an output row), then moves the stage into
// the set piece by piece and reloads it.  The stage load of piece p then has
// 3 + 8 * 2 + 15 = 34 younger operations when it is moved, and the poll
// loads 32 at the end of the step.
//
// Staged scale bytes (kS, every 8 x 8 block whole): a strip's tile byte
// belongs to 8 output rows, one per column, and a wave's 8 strip rows give 8
// consecutive bytes of each.  Written directly that is 64 runs of 8 bytes
// per wave and step.  Instead each wave writes its bytes into an LDS tile of
// the workgroup's 64 output rows x 8 blocks x 8 bytes, and after the next
// step's barrier every thread stores one 8-byte run (the 8 blocks of a
// workgroup run down the columns, so a row's runs are adjacent): one store
// per thread instead of 8, 64-byte runs per row.  Counts per step then: 3 +
// 1 + 8 + 15 = 27 younger operations at a move, 1 + 8 + 16 = 25 at the poll.
template <int p, int kWait>
__device__ __forceinline__ void r2t_move(u32x4 (&cur)[kR2Per], uint32_t& m, __amdgpu_buffer_rsrc_t rx, int voff,
                                         int pstride, uint32_t b0, uint32_t b1, lds_void_t* stage_w) {
  wait_vmcnt<kWait>();
  cur[p] = r8_stage_read<kR2Per, p>(b0, b1);
  const uint32_t h = half_absmax_bits(cur[p]);
  m = m > h ? m : h;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t*)((__attribute__((address_space(3))) char*)stage_w +
                                                             p * kR8StagePiece),
                                           16, voff, p * pstride, 0, kStreamLoad);
  __builtin_amdgcn_sched_barrier(0);
}
template <int kWait, int... P>
__device__ __forceinline__ void r2t_moves(std::integer_sequence<int, P...>, u32x4 (&cur)[kR2Per], uint32_t& m,
                                          __amdgpu_buffer_rsrc_t rx, int voff, int pstride, uint32_t b0, uint32_t b1,
                                          lds_void_t* stage_w) {
  (r2t_move<P, kWait>(cur, m, rx, voff, pstride, b0, b1, stage_w), ...);
}

template <int j>
__device__ __forceinline__ uint32_t r2t_word(const u32x4& v) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

template <int j, bool kS>
__device__ __forceinline__ void r2t_column(const u32x4 (&cur)[kR2Per], double rd, uint32_t sbyte,
                                           __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rsf, int qoff, int soff,
                                           int qstride, int sstride) {
  // column j: element j of every row, row p into element p of the pair of
  // half blocks
  constexpr uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
  uint32_t col[8];
#pragma unroll
  for (int p = 0; p < kR2Per; p += 2)
    col[p / 2] = __builtin_amdgcn_perm(r2t_word<j / 2>(cur[p + 1]), r2t_word<j / 2>(cur[p]), sel);
  const uint32_t c0 = encode_half(u32x4{col[0], col[1], col[2], col[3]}, rd);
  const uint32_t c1 = encode_half(u32x4{col[4], col[5], col[6], col[7]}, rd);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{c0, c1}, rq, qoff, j * qstride, 0);
  if (!kS) __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbyte, rsf, soff, j * sstride, 0);
  __builtin_amdgcn_sched_barrier(0);                   // one column's temporaries at a time
}
template <bool kS, int... J>
__device__ __forceinline__ void r2t_columns(std::integer_sequence<int, J...>, const u32x4 (&cur)[kR2Per], double rd,
                                            uint32_t sbyte, __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rsf,
                                            int qoff, int soff, int qstride, int sstride) {
  (r2t_column<J, kS>(cur, rd, sbyte, rq, rsf, qoff, soff, qstride, sstride), ...);
}

// Staged scale bytes: tile bytes at stile[buf][wave][row][k], row = 8 c + j
// the output row within the workgroup's 64, k the strip row within the block.
constexpr int kSTileBytes = 8 * 64 * 8;                // one buffer

// Thread T stores the 8 bytes of output row T / 8 from block T % 8 of
// tensor t's tile (buffer t & 1) at offset fso (past the extent when the
// block is outside the tensor); t < 0 stores nothing (zero extent).
__device__ __forceinline__ void r2t_flush_scales(const uint8_t* stile, int t, int batch, int64_t hb,
                                                 uint8_t* __restrict__ sf, int fso) {
  const int T = (int)threadIdx.x;
  const u32x2 v = *(const u32x2*)(stile + (t & 1) * kSTileBytes + ((T & 7) * 64 + (T >> 3)) * 8);
  const __amdgpu_buffer_rsrc_t rs = tensor_rsrc(sf, t < 0 ? batch : t, batch, hb / 2);
  __builtin_amdgcn_raw_buffer_store_b64(v, rs, fso, 0, 0);
}

template <bool kS>
__device__ __forceinline__ void r2t_step(const u32x4* __restrict__ x, int t, int batch, int64_t hb, int voff, int qoff,
                                         int soff, int qstride, int sstride, int pstride, u32x4 (&cur)[kR2Per],
                                         uint32_t& tile, uint32_t b0, uint32_t b1, lds_void_t* stage_w, uint32_t* ws,
                                         int G, float* __restrict__ gout, uint32_t* __restrict__ q,
                                         uint8_t* __restrict__ sf, Reg8Shared& sh, uint8_t* stile, int fso) {
  lds_barrier();                                       // t's table is ready; the maxima of t+2 were reduced
  const bool pub = t >= 1 && t + 2 < batch;
  r8_exchange_ops(ws, G, pub ? t + 2 : -1, pub ? r8_red_max(sh.red[(t - 1) & 1]) : 0u, t + 1, t + 1 < batch, sh);
  const double r6 = sh.r6[t & 1];
  const uint32_t sbyte = block_scale_byte(tile, r6);
  const double rd = sh.table[t & 1][sbyte];
  if (kS) {
    r2t_flush_scales(stile, t - 1, batch, hb, sf, fso);   // tensor t-1's tile (the barrier above)
    const int lane = (int)threadIdx.x & 63;
    uint8_t* dst = stile + (t & 1) * kSTileBytes + (wave_id() * 64 + 8 * (lane & 7)) * 8 + (lane >> 3);
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[8 * j] = (uint8_t)sbyte;
    __builtin_amdgcn_sched_barrier(0);
  }
  const __amdgpu_buffer_rsrc_t rq = tensor_rsrc(q, t, batch, hb * 4);
  const __amdgpu_buffer_rsrc_t rsf = tensor_rsrc(sf, t, batch, hb / 2);
  const __amdgpu_buffer_rsrc_t rx = tensor_rsrc(x, t + 4, batch, hb * 16);   // extent zero past the batch
  r2t_columns<kS>(std::make_integer_sequence<int, 8>{}, cur, rd, sbyte, rq, rsf, qoff, soff, qstride, sstride);
  uint32_t m = 0;
  r2t_moves<kS ? kR2Per + 11 : kR2Per + 18>(std::make_integer_sequence<int, kR2Per>{}, cur, m, rx, voff, pstride, b0,
                                            b1, stage_w);
  tile = pair_max(m);                                  // tensor t+3, now in this set
  sh.red[t & 1][wave_id()] = wave_max_u32(m);          // wave-uniform value and address
  wait_vmcnt<kS ? 2 * kR2Per - 7 : 2 * kR2Per>();      // the poll loads of this step have landed
  if (wave_id() == kR8Waves - 1 && t + 1 < batch) r8_table(sh, t + 1, r8_gather(ws, t + 1, G, sh), gout);
}

template <bool kT, bool kS>
__global__ void __launch_bounds__(kR8Data) fused_2d_reg_kernel(const u32x4* __restrict__ x, int batch, int64_t hb,
                                                               int spr, int srows, uint32_t* ws,
                                                               float* __restrict__ gout, uint32_t* __restrict__ q,
                                                               uint8_t* __restrict__ sf) {
  static_assert(kT || !kS, "staged scale bytes are a COLWISE layout");
  __shared__ Reg8Shared sh;
  __shared__ __attribute__((aligned(16))) u32x4 L[kR2Per][kR8Data];
  __shared__ __attribute__((aligned(16))) uint8_t stile[kS ? 2 * kSTileBytes : 16];
  const int G = gridDim.x;
  const int lane = (int)threadIdx.x & 63, wave = wave_id();
  // strip of this thread; strips past the tensor get offsets past every
  // extent (their loads read zeros, their stores are dropped).  Row-major:
  // strip 512 w + i.  COLWISE: wave v of workgroup w takes the block b =
  // 8 w + v of 8 x 8 strips (128 rows x 64 columns; blocks run down the
  // columns), lane l the strip (8 bR + l / 8, 8 bC + l % 8).
  const int pstride = spr * 16;
  int voff, qoff, soff, qstride, sstride, fso = 0;
  if (kT) {
    const int nbr = (srows + 7) / 8, nbc = (spr + 7) / 8;
    const int blk = (int)blockIdx.x * kR8Waves + wave;
    const int br = blk % nbr, bc = blk / nbr;
    const int r = 8 * br + (lane >> 3), c = 8 * bc + (lane & 7);
    const bool in = bc < nbc && r < srows && c < spr;
    const int rows = 16 * srows;
    voff = in ? (r * 16 * spr + c) * 16 : kOnOutside;
    qoff = in ? 8 * c * (rows / 2) + 8 * r : kOnOutside;
    qstride = rows / 2;
    soff = in ? 8 * c * (rows / 16) + r : kOnOutside;
    sstride = rows / 16;
    if (kS) {                                          // this thread's 8-byte run of the staged scales
      const int sb = (int)blockIdx.x * kR8Waves + ((int)threadIdx.x & 7);
      const int sbr = sb % nbr, sbc = sb / nbr;
      fso = sbc < nbc ? (64 * sbc + ((int)threadIdx.x >> 3)) * sstride + 8 * sbr : (int)0x80000000u;
    }
  } else {
    const int st = (int)blockIdx.x * kR8Data + (int)threadIdx.x;
    const int r = st / spr, c = st - r * spr;
    const bool in = r < srows;
    voff = in ? (r * 16 * spr + c) * 16 : kOnOutside;
    qoff = in ? (r * 16 * spr + c) * 4 : kOnOutside;
    qstride = spr * 4;
    // even lanes write the pair's scale byte; odd lanes aim past the extent
    soff = (in && !(lane & 1)) ? (r * 16 * spr + c) / 2 : (int)0x80000000u;
    sstride = spr / 2;
  }
  u32x4 a[kR2Per], b[kR2Per], cc[kR2Per];
  uint32_t ta, tb, tc;
  {
    const __amdgpu_buffer_rsrc_t r0 = tensor_rsrc(x, 0, batch, hb * 16), r1 = tensor_rsrc(x, 1, batch, hb * 16),
                                 r2 = tensor_rsrc(x, 2, batch, hb * 16);
#pragma unroll
    for (int p = 0; p < kR2Per; ++p)
      a[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r0, voff, p * pstride, kStreamLoad));
#pragma unroll
    for (int p = 0; p < kR2Per; ++p)
      b[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r1, voff, p * pstride, kStreamLoad));
#pragma unroll
    for (int p = 0; p < kR2Per; ++p)
      cc[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r2, voff, p * pstride, kStreamLoad));
    __builtin_amdgcn_sched_barrier(0);
  }
  const uint32_t b0 = (uint32_t)(uintptr_t)&L[0][threadIdx.x];
  const uint32_t b1 = b0 + kR8StageSplit * kR8StagePiece;
  lds_void_t* const stage_w =
      (lds_void_t*)(uintptr_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)&L[0][threadIdx.x & ~63]);
  {
    // tensor 3 into the stage.  Row-major: each piece after two stores aimed
    // at zero-extent resources, the memory operations of a step in order;
    // COLWISE steps issue their stores before their loads, so the loads
    // alone give the step's counts
    const __amdgpu_buffer_rsrc_t nq = tensor_rsrc(q, batch, batch, 0), ns = tensor_rsrc(sf, batch, batch, 0);
    const __amdgpu_buffer_rsrc_t rx = tensor_rsrc(x, 3, batch, hb * 16);
#pragma unroll
    for (int p = 0; p < kR2Per; ++p) {
      if (!kT) {
        __builtin_amdgcn_raw_buffer_store_b32(0u, nq, qoff, p * qstride, 0);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)0, ns, soff, p * sstride, 0);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_void_t*)((__attribute__((address_space(3))) char*)stage_w + p * kR8StagePiece), 16, voff,
          p * pstride, 0, kStreamLoad);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  auto step = [&](int tt, u32x4 (&cur)[kR2Per], uint32_t& tile) {
    if (kT)
      r2t_step<kS>(x, tt, batch, hb, voff, qoff, soff, qstride, sstride, pstride, cur, tile, b0, b1, stage_w, ws, G,
                   gout, q, sf, sh, stile, fso);
    else
      r2_step(x, tt, batch, hb, voff, qoff, soff, qstride, sstride, pstride, cur, tile, b0, b1, stage_w, ws, G, gout, q,
              sf, sh);
  };
  sh.red0[0][wave] = set_tile_max(a, ta);
  sh.red0[1][wave] = set_tile_max(b, tb);
  sh.red0[2][wave] = set_tile_max(cc, tc);
  lds_barrier();                                       // maxima of tensors 0..2
  if (wave == kR8Waves - 1) {
    if (lane == 0)
      for (int k = 0; k < 3 && k < batch; ++k) onchip_publish(ws, k, r8_red_max(sh.red0[k]));
    r8_table(sh, 0, onchip_wait(ws, 0, G), gout);
  }
  int t = 0;
  for (; t + 3 <= batch; t += 3) {
    step(t, a, ta);
    step(t + 1, b, tb);
    step(t + 2, cc, tc);
  }
  if (t < batch) step(t, a, ta);
  if (t + 1 < batch) step(t + 1, b, tb);
  if (kS) {
    lds_barrier();                                     // the last tensor's scale tile
    r2t_flush_scales(stile, batch - 1, batch, hb, sf, fso);
  }
  wait_vmcnt<0>();                                     // no stage or poll load still writing LDS at exit
  if (wave != kR8Waves - 1) return;
  // the last workgroup out restores the slots and the counter to zero; every
  // slot store of this workgroup has completed (the wait above)
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

// ------------------------------------------------------------ fused, tensors larger than the chip
// One launch for tensors of nc >= 2 chunks, a chunk being what the on-chip
// kernel holds (D = 512 threads x kPer half blocks per workgroup, one
// workgroup per compute unit).  Per tensor:
//   pass 1: the last three chunks (all of them when nc < 3) load straight
//     into the register sets; every chunk before nc-4 streams through the
//     LDS stage (its maximum taken as it lands, the slot reloaded with the
//     next chunk), and chunk nc-4 stays in the stage;
//   exchange: wave 7 publishes the workgroup's maximum and waits for the
//     tensor's amax, then builds the table;
//   pass 2: the encode walks the chunks in the order nc-3, nc-2, nc-1, nc-4,
//     nc-5, ..., 0: the three register sets, then the stage, then the
//     chunks read a second time.  Each register set, once encoded, reloads
//     with the next chunk to re-read, so up to three re-reads are in flight
//     while the others encode (moving each re-read through the one stage
//     kept only one in flight; 0.083 -> 0.082 ms on 16384 x 7168: the
//     stores of the encodes share the 63 memory operations a wave may have
//     outstanding, so the extra re-reads in flight are few).
// So four chunks are read once and the others twice, newest first (the most
// recently read data is the likeliest to still be in the last-level cache);
// a tensor of at most four chunks is read once.
template <int kPer>
__device__ __forceinline__ void big_load_set(u32x4 (&R)[kPer], __amdgpu_buffer_rsrc_t rs, int voff) {
#pragma unroll
  for (int p = 0; p < kPer; ++p)
    R[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, p * kR8StagePiece, kStreamLoad));
}

template <int kPer>
__device__ __forceinline__ void big_stage_issue(__amdgpu_buffer_rsrc_t rs, lds_void_t* stage_w, int voff) {
#pragma unroll
  for (int p = 0; p < kPer; ++p)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_void_t*)((__attribute__((address_space(3))) char*)stage_w + p * kR8StagePiece), 16, voff,
        p * kR8StagePiece, 0, kStreamLoad);
}

// Pass 1 over one chunk in the stage: the maximum of each piece as it lands
// (the load of piece p has kPer - 1 younger loads: the other pieces), then
// the slot reloaded from `next` at voff_next.
template <int kPer, int p>
__device__ __forceinline__ void big_stage_piece(uint32_t& m, uint32_t b0, uint32_t b1, __amdgpu_buffer_rsrc_t next,
                                                lds_void_t* stage_w, int voff_next) {
  wait_vmcnt<kPer - 1>();
  const u32x4 v = r8_stage_read<kPer, p>(b0, b1);
  const uint32_t h = half_absmax_bits(v);
  m = m > h ? m : h;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(next, (lds_void_t*)((__attribute__((address_space(3))) char*)stage_w +
                                                               p * kR8StagePiece),
                                           16, voff_next, p * kR8StagePiece, 0, kStreamLoad);
  __builtin_amdgcn_sched_barrier(0);
}
template <int kPer, int... P>
__device__ __forceinline__ void big_stage_chunk(std::integer_sequence<int, P...>, uint32_t& m, uint32_t b0, uint32_t b1,
                                                __amdgpu_buffer_rsrc_t next, lds_void_t* stage_w, int voff_next) {
  (big_stage_piece<kPer, P>(m, b0, b1, next, stage_w, voff_next), ...);
}
template <int kPer, int p>
__device__ __forceinline__ void big_stage_piece_max(uint32_t& m, uint32_t b0, uint32_t b1) {
  const uint32_t h = half_absmax_bits(r8_stage_read<kPer, p>(b0, b1));
  m = m > h ? m : h;
}
template <int kPer, int... P>
__device__ __forceinline__ uint32_t big_stage_max(std::integer_sequence<int, P...>, uint32_t b0, uint32_t b1) {
  uint32_t m = 0;
  (big_stage_piece_max<kPer, P>(m, b0, b1), ...);
  return m;
}

// Largest magnitude bits over a register set's pieces (pass 2 takes the
// block maxima again as it encodes, so none are kept here).
template <int kPer>
__device__ __forceinline__ uint32_t big_set_max(const u32x4 (&R)[kPer]) {
  uint32_t m = 0;
#pragma unroll
  for (int p = 0; p < kPer; ++p) {
    const uint32_t h = half_absmax_bits(R[p]);
    m = m > h ? m : h;
  }
  return m;
}

// Chunk held by register set s (0, 1, 2) after pass 1: the last
// nreg = min(nc, 3) chunks in order.
__device__ __forceinline__ int big_chunk(int s, int nc) {
  const int nreg = nc < 3 ? nc : 3;
  return nc - nreg + s;
}

// Pass 2: encode piece p of chunk co (block maximum taken here), store its
// codes and scale byte, then reload the freed registers with piece p of chunk
// cn (cn < 0: nothing more to read).  The compiler places the wait for the
// reload before the piece's next use.
template <int kPer, int p>
__device__ __forceinline__ void big_encode_piece(u32x4 (&X)[kPer], int co, int cn, int cbytes, double r6,
                                                 const double* table, __amdgpu_buffer_rsrc_t rx,
                                                 __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rsf, int voff,
                                                 int qoff, int soff) {
  const uint32_t sbyte = block_scale_byte(pair_max(half_absmax_bits(X[p])), r6);
  const uint32_t code = encode_half(X[p], table[sbyte]);
  __builtin_amdgcn_raw_buffer_store_b32(code, rq, qoff + co * (cbytes / 4), p * kR8Data * 4, kStreamLoad);
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbyte, rsf, soff + co * (cbytes / 32), p * (kR8Data / 2),
                                       0);
  if (cn >= 0)
    X[p] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, voff + cn * cbytes, p * kR8StagePiece, kStreamLoad));
}
template <int kPer, int... P>
__device__ __forceinline__ void big_encode_set(std::integer_sequence<int, P...>, u32x4 (&X)[kPer], int co, int cn,
                                               int cbytes, double r6, const double* table,
                                               __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t rq,
                                               __amdgpu_buffer_rsrc_t rsf, int voff, int qoff, int soff) {
  (big_encode_piece<kPer, P>(X, co, cn, cbytes, r6, table, rx, rq, rsf, voff, qoff, soff), ...);
}

// Pass 2 for the stage's chunk co (its loads landed in pass 1).
template <int kPer, int p>
__device__ __forceinline__ void big_encode_stage_piece(int co, int cbytes, double r6, const double* table,
                                                       __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rsf,
                                                       int qoff, int soff, uint32_t b0, uint32_t b1) {
  const u32x4 v = r8_stage_read<kPer, p>(b0, b1);
  const uint32_t sbyte = block_scale_byte(pair_max(half_absmax_bits(v)), r6);
  const uint32_t code = encode_half(v, table[sbyte]);
  __builtin_amdgcn_raw_buffer_store_b32(code, rq, qoff + co * (cbytes / 4), p * kR8Data * 4, kStreamLoad);
  __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sbyte, rsf, soff + co * (cbytes / 32), p * (kR8Data / 2),
                                       0);
}
template <int kPer, int... P>
__device__ __forceinline__ void big_encode_stage(std::integer_sequence<int, P...>, int co, int cbytes, double r6,
                                                 const double* table, __amdgpu_buffer_rsrc_t rq,
                                                 __amdgpu_buffer_rsrc_t rsf, int qoff, int soff, uint32_t b0,
                                                 uint32_t b1) {
  (big_encode_stage_piece<kPer, P>(co, cbytes, r6, table, rq, rsf, qoff, soff, b0, b1), ...);
}

template <int kPer>
__global__ void __launch_bounds__(kR8Data) fused_big_kernel(const u32x4* __restrict__ x, int batch, int64_t hb,
                                                            uint32_t* ws, float* __restrict__ gout,
                                                            uint32_t* __restrict__ q, uint8_t* __restrict__ sf) {
  static_assert(kPer % 2 == 0 && kPer <= kR8MaxPer, "pieces in pairs, within the register budget");
  __shared__ Reg8Shared sh;
  __shared__ __attribute__((aligned(16))) u32x4 L[kPer][kR8Data];
  const int G = gridDim.x;
  const int lane = (int)threadIdx.x & 63, wave = wave_id();
  const int64_t chunk_hb = (int64_t)G * kPer * kR8Data;
  const int nc = (int)((hb + chunk_hb - 1) / chunk_hb);          // >= 4; hb * 16 < 2^31 (the host checks both)
  const int cbytes = (int)(chunk_hb * 16);
  const int voff = ((int)blockIdx.x * kPer * kR8Data + (int)threadIdx.x) * 16;
  const int qoff = voff / 4;
  // even lanes write the pair's scale byte; odd lanes aim past the extent
  const int soff = (lane & 1) ? (int)0x80000000u : voff / 32;
  const uint32_t b0 = (uint32_t)(uintptr_t)&L[0][threadIdx.x];
  const uint32_t b1 = b0 + kR8StageSplit * kR8StagePiece;
  lds_void_t* const stage_w =
      (lds_void_t*)(uintptr_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uintptr_t)&L[0][threadIdx.x & ~63]);
  const __amdgpu_buffer_rsrc_t none = tensor_rsrc(x, batch, batch, 0);
  for (int t = 0; t < batch; ++t) {
    const __amdgpu_buffer_rsrc_t rx = tensor_rsrc(x, t, batch, hb * 16);
    const __amdgpu_buffer_rsrc_t rq = tensor_rsrc(q, t, batch, hb * 4);
    const __amdgpu_buffer_rsrc_t rsf = tensor_rsrc(sf, t, batch, hb / 2);
    u32x4 a[kPer], b[kPer], c[kPer];
    // ---- pass 1
    big_load_set<kPer>(a, rx, voff + big_chunk(0, nc) * cbytes);
    big_load_set<kPer>(b, nc >= 2 ? rx : none, voff + big_chunk(1, nc) * cbytes);
    big_load_set<kPer>(c, nc >= 3 ? rx : none, voff + big_chunk(2, nc) * cbytes);
    __builtin_amdgcn_sched_barrier(0);
    big_stage_issue<kPer>(nc >= 4 ? rx : none, stage_w, voff);   // chunk 0 (nc - 4 when nc = 4)
    // the register sets' maxima while the stage's first chunk streams in (its
    // kPer loads are the youngest), not after the last load of pass 1 lands
    wait_vmcnt<kPer>();
    uint32_t m = max(max(big_set_max<kPer>(a), big_set_max<kPer>(b)), big_set_max<kPer>(c));
    for (int k = 0; k + 4 < nc; ++k)                    // chunks 0..nc-5 pass through; chunk nc-4 stays
      big_stage_chunk<kPer>(std::make_integer_sequence<int, kPer>{}, m, b0, b1, rx, stage_w, voff + (k + 1) * cbytes);
    wait_vmcnt<0>();                                    // chunk nc-4 has landed
    const uint32_t ms = big_stage_max<kPer>(std::make_integer_sequence<int, kPer>{}, b0, b1);
    m = m > ms ? m : ms;
    sh.red0[0][wave] = wave_max_u32(m);
    lds_barrier();                                      // every wave's maximum of tensor t
    // ---- exchange
    if (wave == kR8Waves - 1) {
      if (lane == 0) onchip_publish(ws, t, r8_red_max(sh.red0[0]));
      r8_table(sh, 0, onchip_wait(ws, t, G), gout + t);
    }
    lds_barrier();                                      // the table of tensor t
    // ---- pass 2
    const double r6 = sh.r6[0];
    const double* table = sh.table[0];
    constexpr auto pieces = std::make_integer_sequence<int, kPer>{};
    // the register sets first, each reloading with the next chunk to re-read
    // (nc-5, nc-6, ..., 0); then the stage's chunk; then the re-read chunks
    // in the sets in turn.  All counts are uniform.
    int nxt = nc - 5;
    int ca = -1, cb = -1, cc = -1;                      // chunk each set holds next (-1: none)
    big_encode_set<kPer>(pieces, a, big_chunk(0, nc), nxt, cbytes, r6, table, rx, rq, rsf, voff, qoff, soff);
    ca = nxt--;
    if (nc >= 2) {
      big_encode_set<kPer>(pieces, b, big_chunk(1, nc), nxt, cbytes, r6, table, rx, rq, rsf, voff, qoff, soff);
      cb = nxt--;
    }
    if (nc >= 3) {
      big_encode_set<kPer>(pieces, c, big_chunk(2, nc), nxt, cbytes, r6, table, rx, rq, rsf, voff, qoff, soff);
      cc = nxt--;
    }
    if (nc >= 4) big_encode_stage<kPer>(pieces, nc - 4, cbytes, r6, table, rq, rsf, qoff, soff, b0, b1);
    while (ca >= 0) {
      big_encode_set<kPer>(pieces, a, ca, nxt, cbytes, r6, table, rx, rq, rsf, voff, qoff, soff);
      ca = nxt >= 0 ? nxt-- : -1;
      if (cb < 0) break;
      big_encode_set<kPer>(pieces, b, cb, nxt, cbytes, r6, table, rx, rq, rsf, voff, qoff, soff);
      cb = nxt >= 0 ? nxt-- : -1;
      if (cc < 0) break;
      big_encode_set<kPer>(pieces, c, cc, nxt, cbytes, r6, table, rx, rq, rsf, voff, qoff, soff);
      cc = nxt >= 0 ? nxt-- : -1;
    }
    wait_vmcnt<0>();
    lds_barrier();                                      // the stage and the table are free for the next tensor
  }
  if (wave != kR8Waves - 1) return;
  // the last workgroup out restores the slots and the counter to zero; every
  // slot store of this workgroup has completed (its wait returned)
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
// The bf16 output is stored non-temporal: written once and not read back
// here, its lines then do not sit dirty in L2 and the last-level cache,
// where the next kernel's reads would have to write them back first.
// Measured with the fused quantize alternating with this kernel on
// 64 x 2048 x 7168: dequantize 0.406 -> 0.400 ms, the quantize after it
// 0.438 -> 0.415 ms.
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
    for (int u = 0; u < kU; ++u)
      __builtin_nontemporal_store(dequant_half(c[u], e4m3_value(s[u]), g), yt + i + u * step);
  }
  for (; i < hb_per_tensor; i += step) __builtin_nontemporal_store(dequant_half(qt[i], e4m3_value(st[i >> 1]), g), yt + i);
}

// Clears n words of scratch (the exchange header of a workspace whose
// contents are not guaranteed, before a co-resident launch uses it).
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

// Half blocks per data thread for the on-chip FUSED launch: the smallest
// even count that covers a tensor with at most one workgroup per CU, or 0
// when the tensor is too large to hold on chip (the streaming launch runs
// then).
int onchip_per_thread(int64_t hb_per_tensor) {
  if (hb_per_tensor <= 0) return 0;
  const int64_t cus = nvfp4host::num_cus();
  if (cus > kR8PollSlots || cus > (int64_t)kTensorWords) return 0;   // one exchange slot per workgroup
  const int64_t cap = cus * kR8Data;
  int64_t per = (hb_per_tensor + cap - 1) / cap;
  per += per & 1;                                       // pieces pair up in the block-maximum words
  return per <= kR8MaxPer ? (int)per : 0;
}

// Chunks of fused_big_kernel for a tensor (one workgroup per CU, kR8MaxPer
// half blocks per data thread), or 0 when it does not apply: a tensor that
// fits on chip in one chunk, or one whose byte offsets would not fit the
// 32-bit buffer offsets.
int big_chunks(int64_t hb_per_tensor) {
  if (hb_per_tensor <= 0) return 0;
  const int64_t cus = nvfp4host::num_cus();
  if (cus > kR8PollSlots || cus > (int64_t)kTensorWords) return 0;
  const int64_t chunk = cus * kR8MaxPer * kR8Data;
  const int64_t nc = (hb_per_tensor + chunk - 1) / chunk;
  if (nc < 2 || nc * chunk * 16 >= (INT64_C(1) << 31)) return 0;
  return (int)nc;
}

// Launches a kernel whose workgroups wait for one another (bounded waits):
// the grid is at most one round of resident workgroups (the caller sizes it
// from the device's compute units and the kernel's occupancy), so on a
// device not filled by other persistent kernels every workgroup starts at
// once.  A plain launch: a cooperative one guarantees the same residency but
// costs about 16 us more per launch on this device; if some workgroup did
// not become resident in time, the waits give up, g becomes NaN and
// nvfp4_quantize_status reports it.
nvfp4_status launch_resident(const void* fn, int grid, int block, void** args, hipStream_t s) {
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)block), args, 0, s);
  if (e != hipSuccess) {
    nvfp4host::set_hip_error(e);
    return NVFP4_EHIP;
  }
  return NVFP4_OK;
}

}  // namespace

namespace nvfp4host {

// Scratch bytes of quantize_2d_onchip for a batch (the exchange header).
size_t quantize_2d_onchip_ws_bytes(int64_t batch) {
  return batch <= 0 ? 0 : (fused_header_bytes(batch) + 255) & ~(size_t)255;
}

// 2D quantize (one E4M3 scale per 16 x 16 tile; outputs row-major, or
// transposed with colwise) of batch tensors [rows][cols] in one launch of
// fused_2d_reg_kernel when a tensor's 16-row x 8-column strips fit on the
// chip, one per thread: every input byte is read once.  ENOTSUP when they do
// not (the caller then runs its two-pass path).  The exchange header in ws is
// cleared first, so the scratch needs no preparation.  The shape and
// pointers are validated by the caller (rows % 16 == 0, cols % 16 == 0).
nvfp4_status quantize_2d_onchip(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, bool colwise, uint8_t* q,
                                uint8_t* sf, float* g, void* ws, hipStream_t s) {
  if (batch <= 0 || rows <= 0 || cols <= 0) return NVFP4_ENOTSUP;
  const int64_t cus = num_cus();
  if (cus > (int64_t)kTensorWords) return NVFP4_ENOTSUP;   // one exchange slot per workgroup
  const int64_t srows = rows / 16, spr = cols / 8;
  // one 16-row strip per thread of fused_2d_reg_kernel (512 per workgroup;
  // COLWISE: in blocks of 8 x 8 strips, one per wave)
  const int64_t G = colwise ? (((srows + 7) / 8) * ((spr + 7) / 8) + kR8Waves - 1) / kR8Waves
                            : (srows * spr + kR8Data - 1) / kR8Data;
  if (G > cus || G > kR8PollSlots) return NVFP4_ENOTSUP;
  if (rows * cols * 2 >= (INT64_C(1) << 31)) return NVFP4_ENOTSUP;   // 32-bit buffer offsets
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
  // COLWISE with every 8 x 8 block whole stages its scale bytes
  const bool staged = colwise && srows % 8 == 0 && spr % 8 == 0;
  const void* fn = staged ? (const void*)fused_2d_reg_kernel<true, true>
                   : colwise ? (const void*)fused_2d_reg_kernel<true, false>
                             : (const void*)fused_2d_reg_kernel<false, false>;
  return launch_resident(fn, (int)G, kR8Data, args, s);
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

}  // extern "C"

namespace {

// Host validation of nvfp4_quantize's arguments (nothing is launched).
// Returns OK, or OK with *empty set when there is nothing to do.
nvfp4_status quantize_validate(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, const uint8_t* q,
                               const uint8_t* sf, const float* g, const void* workspace, size_t workspace_bytes,
                               uint32_t flags, bool* empty) {
  *empty = false;
  nvfp4_status st = check_shape(batch, rows, cols);
  if (st) return st;
  if (flags != NVFP4_TWO_KERNEL && flags != NVFP4_FUSED) return NVFP4_ENOTSUP;
  if (batch == 0) {
    *empty = true;
    return NVFP4_OK;
  }
  if (!g) return NVFP4_EINVAL;
  const int64_t n = rows * cols;
  if (n > 0 && (!x || !q || !sf)) return NVFP4_EINVAL;
  if (!nvfp4host::aligned16(x) || !nvfp4host::aligned16(q) || !nvfp4host::aligned16(sf) || !nvfp4host::aligned16(g))
    return NVFP4_EALIGN;
  if (!workspace || workspace_bytes < nvfp4_quantize_workspace_bytes(batch, rows, cols)) return NVFP4_EWORKSPACE;
  if (!nvfp4host::aligned16(workspace)) return NVFP4_EALIGN;
  return nvfp4host::check_device();
}

// The launches of nvfp4_quantize, arguments already validated.
nvfp4_status quantize_launch(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sf,
                             float* g, void* workspace, uint32_t flags, hipStream_t s) {
  const int64_t n = rows * cols;
  const int64_t hb = n / 8;
  if (flags == NVFP4_FUSED) {
    const int onchip_per = onchip_per_thread(hb);
    const u32x4* xa = (const u32x4*)x;
    int bt = (int)batch;
    uint32_t* ws = (uint32_t*)workspace;
    uint32_t* qa = (uint32_t*)q;
    void* args[] = {&xa, &bt, (void*)&hb, &ws, &g, &qa, &sf};
    if (onchip_per > 0) {
      const int64_t slice = (int64_t)onchip_per * kR8Data;
      const int G = (int)((hb + slice - 1) / slice);
      const void* fns[kR8MaxPer / 2] = {
          (const void*)fused_reg8_kernel<2>,  (const void*)fused_reg8_kernel<4>,  (const void*)fused_reg8_kernel<6>,
          (const void*)fused_reg8_kernel<8>,  (const void*)fused_reg8_kernel<10>, (const void*)fused_reg8_kernel<12>,
          (const void*)fused_reg8_kernel<14>,
      };
      return launch_resident(fns[onchip_per / 2 - 1], G, kR8Data, args, s);
    }
    if (big_chunks(hb) > 0)
      return launch_resident((const void*)fused_big_kernel<kR8MaxPer>, (int)nvfp4host::num_cus(), kR8Data, args, s);
    return launch_resident((const void*)fused_quantize_kernel, fused_grid(hb), kThreads, args, s);
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

// ------------------------------------------------------------ allocation-free quantize
// The workspace of nvfp4_quantize_noalloc: a fixed device array, one copy
// per GPU, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it only stands for the symbol): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is cached per device.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

nvfp4_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    nvfp4host::set_hip_error(e);
    return NVFP4_EHIP;
  }
  if (dev < 0 || dev >= kMaxScratchDevices) return NVFP4_ENOTSUP;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      nvfp4host::set_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return NVFP4_EHIP;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);   // every caller stores the same address
  }
  *out = p;
  return NVFP4_OK;
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_quantize(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sf,
                            float* g, void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  bool empty = false;
  const nvfp4_status st =
      quantize_validate(x, batch, rows, cols, q, sf, g, workspace, workspace_bytes, flags, &empty);
  if (st || empty) return st;
  return quantize_launch(x, batch, rows, cols, q, sf, g, workspace, flags, (hipStream_t)stream);
}

nvfp4_status nvfp4_quantize_noalloc(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint8_t* q,
                                    uint8_t* sf, float* g, uint32_t flags, void* stream) {
  nvfp4_status st = check_shape(batch, rows, cols);
  if (st) return st;
  if (batch > 0 && nvfp4_quantize_workspace_bytes(batch, rows, cols) > kNoAllocScratchBytes) return NVFP4_EWORKSPACE;
  void* ws = nullptr;
  if (batch > 0 && (st = scratch_for_current_device(&ws))) return st;
  bool empty = false;
  st = quantize_validate(x, batch, rows, cols, q, sf, g, ws, kNoAllocScratchBytes, flags, &empty);
  if (st || empty) return st;
  hipStream_t s = (hipStream_t)stream;
  if (flags == NVFP4_FUSED) {
    // the exchange words start at zero whatever an earlier call left (a fill
    // kernel, not a memset, so the call can sit in a captured graph)
    const int64_t words = (int64_t)(fused_header_bytes(batch) / 4);
    zero_words_kernel<<<(unsigned)std::min<int64_t>((words + kThreads - 1) / kThreads, 1024), kThreads, 0, s>>>(
        (uint32_t*)ws, words);
    NVFP4_LAUNCH_CHECK();
  }
  return quantize_launch(x, batch, rows, cols, q, sf, g, ws, flags, s);
}

uint32_t nvfp4_set_wait_limit(uint32_t polls) {
  uint32_t prev = kDefaultWaitLimit;
  if (hipMemcpyFromSymbol(&prev, HIP_SYMBOL(g_wait_limit), sizeof(prev)) != hipSuccess) prev = kDefaultWaitLimit;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_wait_limit), &polls, sizeof(polls)) != hipSuccess) return prev;
  return prev;
}

nvfp4_status nvfp4_quantize_status(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < sizeof(FusedHeader)) return NVFP4_EWORKSPACE;
  nvfp4_status st = nvfp4host::check_device();
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipStreamSynchronize(s);
  FusedHeader h{};
  if (e == hipSuccess) e = hipMemcpy(&h, workspace, sizeof(h), hipMemcpyDeviceToHost);
  if (e == hipSuccess && h.error) {
    const uint32_t zero = 0;
    e = hipMemcpy((char*)workspace + offsetof(FusedHeader, error), &zero, sizeof(zero), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    nvfp4host::set_hip_error(e);
    return NVFP4_EHIP;
  }
  return h.error ? NVFP4_ETIMEOUT : NVFP4_OK;
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
