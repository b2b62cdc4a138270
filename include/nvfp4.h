/*
 * libnvfp4 -- NVFP4 two-level microscaling on AMD Instinct MI355X (gfx950).
 *
 * NVFP4 stores each value as a 4-bit E2M1 float (1 sign, 2 exponent, 1
 * mantissa bit: +-0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6); 16 consecutive
 * values share one E4M3 block scale and the whole tensor has one FP32 scale,
 * about 4.5 bits (0.5625 bytes) per value.  Sources: axbrief.com, "NVFP4: how
 * NVIDIA pre-trained a 12B model on 10 trillion tokens", section "E2M1 format
 * and two-level scaling"; iwan.kr, "NVIDIA shrank GLM-5.2 to 4 bits", section 3
 * "Terminology: quantization and NVFP4"; theddari.com, "What is FP4
 * quantization? KV cache in 4 bits", format-comparison table.
 *
 * Numeric recipe (the pages leave the formulas open; this is the plain
 * reading that maps each block's amax onto the E2M1 maximum):
 *   g  = RN32(amax / 2688)                 2688 = 6 (E2M1 max) * 448 (E4M3 max)
 *   s  = E4M3_RNE_SAT(RN32(bamax / RN32(6 g)))            (0 when 6g == 0)
 *   code = sign(x) << 3 | E2M1_RNE_SAT(RN32(|x| / RN32(s g)))
 *          (a signed zero when s g == 0)
 *   value = bf16_RNE(RN32((E2M1(code) * s) * g))
 * RN32 is one IEEE binary32 rounding to nearest-even.  E4M3 is OCP E4M3FN
 * (max 448, byte 0x7F never produced).  Ties on both grids go to the even
 * code.  Results are bit-exact across every entry point and launch mode.
 *
 * Layouts (row-major, contiguous, no swizzle):
 *   x  [batch][rows][cols] bf16 bit patterns (uint16_t), cols % 16 == 0
 *   q  [batch][rows][cols/2] uint8, element 2j in the LOW nibble of byte j
 *   sf [batch][rows][cols/16] uint8 E4M3 block-scale bytes
 *   g  [batch] float, one tensor scale per batch item
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates or frees device memory.  Every call enqueues
 *     kernels on `stream` (a hipStream_t, NULL = the default stream) and
 *     returns without synchronizing, except the two calls documented as
 *     synchronous (nvfp4_quantize_status, nvfp4_set_wait_limit).
 *     Device-side faults surface at the caller's next sync.
 *   - Arguments are validated on the host before any launch.  On an error
 *     code nothing is launched and no output byte is written.
 *   - Inputs must be finite (not checked on the device; non-finite inputs give
 *     unspecified codes but never out-of-bounds accesses).
 *   - Tensor base pointers must be 16-byte aligned (NVFP4_EALIGN otherwise).
 *   - Sizes are int64_t; negative sizes are NVFP4_EINVAL, zero sizes are a
 *     successful no-op.
 *   - Thread-safe; the only global state is a once-per-device architecture
 *     check, a per-thread last-HIP-error slot and the per-device wait limit
 *     of nvfp4_set_wait_limit.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t nvfp4_status;

enum {
  NVFP4_OK = 0,
  NVFP4_EINVAL = -1,     /* null pointer, bad dimension, cols % 16 != 0, range */
  NVFP4_EALIGN = -2,     /* a tensor base pointer is not 16-byte aligned */
  NVFP4_EWORKSPACE = -3, /* workspace missing or smaller than required */
  NVFP4_ENOTSUP = -4,    /* current device is not gfx950, or unsupported flag */
  NVFP4_EHIP = -5,       /* a HIP runtime call failed; see nvfp4_last_hip_error */
  NVFP4_ETIMEOUT = -6    /* nvfp4_quantize_status: a FUSED launch's bounded wait gave up */
};

/* Launch modes of nvfp4_quantize. */
enum {
  NVFP4_TWO_KERNEL = 0,  /* pass 1: per-tensor amax kernel; pass 2: encode kernel */
  NVFP4_FUSED = 1        /* one launch of co-resident workgroups, amax then encode */
};

#define NVFP4_ABI_VERSION 1
int32_t nvfp4_abi_version(void);

/* Human-readable name of a status code (static storage, never NULL). */
const char* nvfp4_status_string(nvfp4_status status);

/* hipError_t of the last NVFP4_EHIP returned on the calling thread (0 if none). */
int32_t nvfp4_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Quantize: bf16 -> NVFP4 with the tensor scale computed from the tensor's
 * own amax (activations; weights).  Two-level scaling of axbrief.com, "NVFP4:
 * how NVIDIA pre-trained a 12B model on 10 trillion tokens", section "E2M1
 * format and two-level scaling": the FP32 tensor scale sets the overall range
 * and the E4M3 block scale maps each 16-value block's amax near the E2M1 max.
 *
 * x:  [batch][rows][cols] bf16 (read)     q:  [batch][rows][cols/2] (written)
 * sf: [batch][rows][cols/16] (written)    g:  [batch] float (written)
 * workspace: device scratch of at least nvfp4_quantize_workspace_bytes(...)
 *   bytes, caller-owned.  It must be zero-filled once when allocated; the
 *   library leaves it ready for the next call.  Calls that share one
 *   workspace must be ordered on one stream.
 * flags: NVFP4_TWO_KERNEL or NVFP4_FUSED (same bytes either way).
 * Errors: EINVAL (null pointer with nonzero size, negative size, cols % 16),
 *   EALIGN, EWORKSPACE, ENOTSUP (unknown flag / not gfx950), EHIP.
 * FUSED runs every workgroup of one launch through a cross-workgroup
 * exchange of maxima; the grid is at most one round of resident workgroups
 * (one per compute unit for tensors under 2 GiB), so FUSED calls
 * must not overlap in time with other kernels that occupy the whole device
 * and wait for one another (such as a FUSED call on another stream).  Each
 * wait is bounded (see nvfp4_set_wait_limit).  A wait that gives up -- which
 * a launch on an otherwise idle device never needs -- does not fault: it writes NaN
 * for the tensor scale g of that tensor, leaves its codes and scale bytes
 * unspecified (in bounds), and sets an error word in the workspace that
 * nvfp4_quantize_status reports.
 * ------------------------------------------------------------------------ */
size_t nvfp4_quantize_workspace_bytes(int64_t batch, int64_t rows, int64_t cols);

nvfp4_status nvfp4_quantize(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                            uint8_t* q, uint8_t* sf, float* g,
                            void* workspace, size_t workspace_bytes,
                            uint32_t flags, void* stream);

/* nvfp4_quantize for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and bytes, with the workspace in a
 * fixed 1 MiB device array inside the library (one copy per GPU, held until
 * the process ends) instead of a caller buffer.  Allocates nothing.
 * Limit: nvfp4_quantize_workspace_bytes(batch, rows, cols) <= 1 MiB, i.e.
 * batch <= 101; larger batches return NVFP4_EWORKSPACE.  Every call on one
 * GPU shares that array: calls that overlap in time on one GPU (different
 * streams, or threads without ordering) race and must not be made.  A FUSED
 * call first clears the array's exchange words with a small fill kernel.  A
 * FUSED wait that gives up leaves NaN in g, as for nvfp4_quantize.
 * Errors: as nvfp4_quantize (EWORKSPACE: batch above the limit). */
nvfp4_status nvfp4_quantize_noalloc(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                    uint8_t* q, uint8_t* sf, float* g, uint32_t flags, void* stream);

/* Reports whether a FUSED nvfp4_quantize on this workspace had a bounded
 * wait give up since the last report: synchronizes `stream` (the one the
 * calls ran on), reads the workspace's error word, clears it, and returns
 * NVFP4_ETIMEOUT if it was set (the affected tensors' g are NaN), else
 * NVFP4_OK.  The only entry point that synchronizes or copies to the host.
 * Errors: EWORKSPACE (null or too small), ENOTSUP, EHIP. */
nvfp4_status nvfp4_quantize_status(void* workspace, size_t workspace_bytes, void* stream);

/* Sets the number of polls after which every bounded wait of the
 * FUSED and single-launch 2D kernels gives up, on the current device; returns the previous
 * value (default 2^24, seconds of polling).  For tests and diagnostics: 0
 * makes every wait give up at once (every kernel still runs to its end), so
 * the timeout path can be exercised without a stalled grid.  Synchronous. */
uint32_t nvfp4_set_wait_limit(uint32_t polls);

/* Quantize with caller-supplied tensor scales g[batch] (read, not written):
 * a static or calibrated scale, no amax pass (theddari.com, "What is FP4
 * quantization? KV cache in 4 bits", checklist item 2: KV scales come from
 * calibration).  g must hold finite values >= 0. */
nvfp4_status nvfp4_quantize_with_scale(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                                       const float* g, uint8_t* q, uint8_t* sf, void* stream);

/* Dequantize NVFP4 -> bf16: the runtime restores approximate values from the
 * stored scales (omidsaffari.com, "LLM quantization guide", section "What is
 * LLM quantization").  y: [batch][rows][cols] bf16 (written). */
nvfp4_status nvfp4_dequantize(const uint8_t* q, const uint8_t* sf, const float* g,
                              int64_t batch, int64_t rows, int64_t cols,
                              uint16_t* y, void* stream);

/* ------------------------------------------------------------------------
 * NVFP4 KV cache (theddari.com, "What is FP4 quantization? KV cache in 4
 * bits", sections "KV cache size example" and "how does 4-bit KV change
 * inference cost": K and V are stored in NVFP4, 0.5625 bytes per value, and
 * decoding re-reads the cache every step).  Each (layer, kv-head, token) K or
 * V vector of head_dim values is one row of head_dim/16 blocks quantized with
 * the (layer, head) tensor scale, which the caller fixes at cache creation.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t layers, kv_heads, head_dim;    /* head_dim % 16 == 0 */
  int64_t capacity;                      /* maximum tokens */
  uint8_t* k;                            /* [layers][kv_heads][capacity][head_dim/2]  */
  uint8_t* v;                            /* [layers][kv_heads][capacity][head_dim/2]  */
  uint8_t* k_sf;                         /* [layers][kv_heads][capacity][head_dim/16] */
  uint8_t* v_sf;                         /* [layers][kv_heads][capacity][head_dim/16] */
  const float* k_g;                      /* [layers][kv_heads] tensor scales (device) */
  const float* v_g;                      /* [layers][kv_heads] tensor scales (device) */
} nvfp4_kv_cache;

/* Bytes of codes + block scales held by the cache:
 * capacity * 2 * layers * kv_heads * head_dim * 0.5625 (tensor scales excluded).
 * Returns 0 for an invalid descriptor. */
size_t nvfp4_kv_bytes(const nvfp4_kv_cache* cache);

/* Append n tokens at positions [start, start+n).  k_new, v_new:
 * [layers][n][kv_heads][head_dim] bf16.  EINVAL if start < 0 or
 * start + n > capacity.  The caller tracks the cache length.  An append
 * writes only the codes and scales of its own token range, so appends of
 * disjoint ranges may run concurrently on different streams. */
nvfp4_status nvfp4_kv_append(const nvfp4_kv_cache* cache, int64_t start, int64_t n,
                             const uint16_t* k_new, const uint16_t* v_new, void* stream);

/* Dequantize tokens [t0, t0+n) of layers [layer0, layer0+nlayers) to bf16:
 * k_out, v_out: [nlayers][kv_heads][n][head_dim] (either may be NULL to skip). */
nvfp4_status nvfp4_kv_read(const nvfp4_kv_cache* cache, int32_t layer0, int32_t nlayers,
                           int64_t t0, int64_t n, uint16_t* k_out, uint16_t* v_out, void* stream);

/* One decode step's attention logits over the first n cached tokens:
 * logits[l][hq][t] = sum_d q[l][hq][d] * Khat[l][hq / (q_heads/kv_heads)][t][d]
 * (unscaled dot products, fp32 accumulation; Khat is the exact dequantized K).
 * q: [layers][q_heads][head_dim] bf16; q_heads a multiple of kv_heads (GQA).
 * logits: [layers][q_heads][n] float.  Relative error of the logits is within
 * fp32 accumulation of the exact fp64 sums.
 * Errors: EINVAL (q_heads not a multiple of kv_heads, n outside
 *   [0, capacity]), ENOTSUP (more than 16 query heads per KV head, (q_heads /
 *   kv_heads) * head_dim above 4096, or head_dim/16 not a power of two up to
 *   64), EALIGN, EHIP. */
nvfp4_status nvfp4_kv_decode_qk(const nvfp4_kv_cache* cache, const uint16_t* q, int32_t q_heads,
                                int64_t n, float* logits, void* stream);

/* One decode step of attention over the first n cached tokens, consuming
 * the NVFP4 cache directly (decoding re-reads the whole cache each step:
 * theddari.com, "What is FP4 quantization? KV cache in 4 bits", section "how
 * does 4-bit KV change inference cost").  For layer l and query head hq
 * (KV head h = hq / (q_heads/kv_heads)):
 *   s_t = scale * sum_d q[l][hq][d] * Khat[l][h][t][d]            (t < n)
 *   out[l][hq][d] = sum_t exp(s_t - max s) Vhat[l][h][t][d] / sum_t exp(s_t - max s)
 * Khat, Vhat are the exact dequantized values; fp32 accumulation, fp32 exp.
 * q: [layers][q_heads][head_dim] bf16; out: [layers][q_heads][head_dim] float.
 * workspace: at least nvfp4_kv_attention_workspace_bytes(cache, q_heads, n)
 *   bytes of device scratch (per-split partial results; no zero-fill needed).
 * head_dim 64, 128 or 256 with up to 16 query heads per KV head runs both
 * contractions on MFMA: K and V decoded exactly to f16, q scaled per head by
 * a power of two (largest element in [2^14, 2^15)) and rounded to f16, which
 * is exact for every element above 2^-28 of the head's largest; P split into
 * f16 hi + lo parts.  head_dim 16 or 32 with 1, 2, 4 or 8 query heads per KV
 * head runs in VALU with bf16 q.
 * Errors: EINVAL (n < 1 or n > capacity, q_heads not a multiple of kv_heads,
 *   non-finite scale, n * head_dim / 2 >= 2^30), ENOTSUP (any other shape),
 *   EWORKSPACE, EALIGN, EHIP. */
size_t nvfp4_kv_attention_workspace_bytes(const nvfp4_kv_cache* cache, int32_t q_heads, int64_t n);

nvfp4_status nvfp4_kv_decode_attention(const nvfp4_kv_cache* cache, const uint16_t* q, int32_t q_heads,
                                       int64_t n, float scale, float* out,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Block-scaled NVFP4 x NVFP4 GEMM for MoE expert linears, weights and
 * activations both NVFP4 (iwan.kr, "NVIDIA shrank GLM-5.2 to 4 bits",
 * section 1; FP4 GEMM speed, axbrief.com, section "36% token efficiency and
 * Blackwell speed"):
 *   C[m][n] = gA * gB * sum_k deq(A)[m][k] * deq(B)[n][k]        (TN, K-major)
 * deq() = E2M1(code) * s, exact in f16 (at most 6 significant bits); fp32
 * accumulation; the tensor scales are applied once in the epilogue.  Both
 * operands use the quantize layout: a_q [M][K/2], a_sf [M][K/16], b_q
 * [N][K/2], b_sf [N][K/16]; a_g, b_g point to one float each (device).
 * c: [M][N] float, fully written (zeros when K == 0).
 * Errors: EINVAL (K % 16 != 0, K > 2^22, negative or too large M / N, null
 *   pointers), EALIGN (a_q, b_q, c not 16-byte aligned, a_g / b_g not
 *   4-byte aligned), ENOTSUP, EHIP.
 * ------------------------------------------------------------------------ */
nvfp4_status nvfp4_gemm(const uint8_t* a_q, const uint8_t* a_sf, const float* a_g,
                        const uint8_t* b_q, const uint8_t* b_sf, const float* b_g,
                        int64_t M, int64_t N, int64_t K, float* c, void* stream);

/* ------------------------------------------------------------------------
 * Grouped block-scaled GEMM for the MoE expert linears (iwan.kr, "NVIDIA
 * shrank GLM-5.2 to 4 bits", section 1: the experts' weights and activations
 * are both NVFP4).  The rows of A are the routed tokens sorted by expert:
 * rows [offsets[e], offsets[e+1]) go through expert e's weight B_e.
 *   C[m][n] = gA * gB[e] * sum_k deq(A)[m][k] * deq(B_e)[n][k]   (m in expert e's rows)
 * a_q [M][K/2], a_sf [M][K/16], a_g: one float (device).
 * b_q [experts][N][K/2], b_sf [experts][N][K/16], b_g [experts] (device).
 * offsets: [experts+1] int32 on the device, non-decreasing from 0 to M; the
 *   kernels clamp them to [0, M], so inconsistent offsets leave rows of C
 *   unwritten but never access memory outside A, B or C.
 * c: [M][N] float; every row inside some expert's range is written.
 * Each expert's rows are computed exactly as nvfp4_gemm computes that
 * expert's slice of A (same tiles, same accumulation order).
 * Errors: EINVAL (experts <= 0, K % 16 != 0, K > 2^22, M / 256 + experts
 *   above 65535, null pointers), EALIGN, ENOTSUP, EHIP.
 * ------------------------------------------------------------------------ */
nvfp4_status nvfp4_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sf, const float* a_g,
                                const uint8_t* b_q, const uint8_t* b_sf, const float* b_g,
                                const int32_t* offsets, int32_t experts,
                                int64_t M, int64_t N, int64_t K, float* c, void* stream);

/* ------------------------------------------------------------------------
 * Quantize variants of the NVFP4 training recipe (axbrief.com, "NVFP4: how
 * NVIDIA pre-trained a 12B model on 10 trillion tokens", section "Four
 * stabilizers for training: from RHT to stochastic rounding"), combinable
 * bit flags:
 *   NVFP4_VAR_COLWISE  quantize x^T (blocks run down x's columns): the
 *                      Dgrad / Wgrad operand layout.  Outputs describe the
 *                      [cols][rows] matrix.  Needs rows % 16 == 0.
 *   NVFP4_VAR_2D       one E4M3 scale per 16 x 16 tile from the tile's amax
 *                      (weights: W and W^T quantize to the same values); the
 *                      byte is written for each of the tile's 16 rows, so sf
 *                      keeps the [R][C/16] layout every consumer reads.
 *                      Needs rows % 16 == 0; not combined with RHT (ENOTSUP).
 *   NVFP4_VAR_RHT      each 16-value block (along the block direction) is
 *                      replaced by H16 (s .* x) / 4 before quantizing: H16
 *                      the Sylvester Hadamard matrix (H[i][j] =
 *                      (-1)^popcount(i & j)), s_j = -1 where bit j of
 *                      rht_signs is set; computed in fp32 as the fast
 *                      Walsh-Hadamard stages h = 1, 2, 4, 8 (pairs (i, i+h)
 *                      with i & h == 0 become (a + b, a - b)), then * 1/4.
 *                      The tensor amax and every quotient use these fp32
 *                      values.
 *   NVFP4_VAR_SR       stochastic element rounding: with lo <= y < hi the
 *                      neighbouring E2M1 magnitudes of y = RN32(|x| / d),
 *                      the code rounds up when u16 / 65536 < (y - lo) /
 *                      (hi - lo) (y >= 6 gives 6).  u16: Philox4x32-10
 *                      (Salmon et al., SC 2011), key (seed, seed >> 32),
 *                      counter (n, n >> 32, 0, 0) with n = i / 8 + offset
 *                      for output element i (row-major index into q's
 *                      values across the batch), 16-bit half i % 2 (low
 *                      first) of word (i % 8) / 2.  Block scales stay
 *                      round-to-nearest.
 * ------------------------------------------------------------------------ */
enum {
  NVFP4_VAR_COLWISE = 1,
  NVFP4_VAR_2D = 2,
  NVFP4_VAR_RHT = 4,
  NVFP4_VAR_SR = 8
};

/* Device scratch for nvfp4_quantize_ex: the single-launch 2D path's
 * exchange words, then per-workgroup partial maxima (no zero-fill needed:
 * the library clears what it relies on, error word included, at the start
 * of each call; a bounded wait of that single launch that gave up is
 * reported by nvfp4_quantize_status on the same workspace until the next
 * nvfp4_quantize_ex call on it).  0 when batch <= 0. */
size_t nvfp4_quantize_ex_workspace_bytes(int64_t batch);

/* Variant quantize of x [batch][rows][cols] bf16 (cols % 16 == 0).  With
 * (R, C) = (rows, cols), or (cols, rows) under COLWISE: q [batch][R][C/2],
 * sf [batch][R][C/16], g [batch] (the tensor scale of the transformed
 * values).  Two passes over x (amax, then encode); 2D without RHT or SR
 * (with or without COLWISE) reads x once in a single launch
 * when a tensor's strips of 16 rows x 8 columns fit on the chip (at most
 * compute units x 512 of them; COLWISE counts blocks of 8 x 8 strips, 8 per
 * compute unit) and a tensor is under 2 GiB, with the same bytes.  variant 0
 * equals nvfp4_quantize bit for bit.
 * Errors: EINVAL (cols % 16 != 0, rows % 16 != 0 with COLWISE or 2D, unknown
 *   variant bits, rht_signs > 0xFFFF, batch > 65535, null pointers), ENOTSUP
 *   (2D with RHT, or the device), EALIGN (x, q not 16-byte aligned; g,
 *   workspace not 4-byte aligned), EWORKSPACE, EHIP. */
nvfp4_status nvfp4_quantize_ex(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint32_t variant,
                               uint32_t rht_signs, uint64_t seed, uint64_t offset, uint8_t* q, uint8_t* sf,
                               float* g, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * MXFP4, the earlier microscaling format: 32 consecutive E2M1 values share
 * one power-of-two scale stored as an E8M0 byte (value 2^(byte - 127), 255
 * is NaN); there is no tensor scale; about 4.25 bits per value (iwan.kr,
 * "NVIDIA shrank GLM-5.2 to 4 bits", section 3 "Terminology"; axbrief.com,
 * "NVFP4: how NVIDIA pre-trained a 12B model on 10 trillion tokens", section
 * "36% token efficiency and Blackwell speed"; theddari.com, "What is FP4
 * quantization? KV cache in 4 bits", format-comparison table).
 * The pages leave the exponent rule open; it is the published Microscaling
 * definition of the format:
 *   X = floor(log2(block amax)) - 2, clamped to [-127, 127]
 *       (an all-zero block takes X = -127); scale byte = X + 127
 *   code = sign(x) << 3 | E2M1_RNE_SAT(RN32(|x| / 2^X))
 *       (values between 6 * 2^X and 8 * 2^X saturate to 6 * 2^X)
 *   value = bf16_RNE(RN32(E2M1(code) * 2^X))
 * Layouts: x [rows][cols] bf16 (cols % 32 == 0; a batch is rows of one
 * matrix, since no state is per tensor), q [rows][cols/2] uint8 (element 2j
 * in the low nibble of byte j, as for NVFP4), sf [rows][cols/32] uint8.
 * ------------------------------------------------------------------------ */

/* Quantize bf16 x to MXFP4 in one pass.  Bit-exact to the recipe above.
 * Errors: EINVAL (cols % 32 != 0, negative sizes, null pointers), EALIGN
 *   (x or q not 16-byte aligned), ENOTSUP, EHIP. */
nvfp4_status nvfp4_mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sf,
                                  void* stream);

/* Dequantize MXFP4 to bf16 y [rows][cols].  Scale byte 255 gives NaN;
 * products beyond bf16's range give +-inf.  Errors as nvfp4_mxfp4_quantize
 * (EALIGN: q or y not 16-byte aligned). */
nvfp4_status nvfp4_mxfp4_dequantize(const uint8_t* q, const uint8_t* sf, int64_t rows, int64_t cols, uint16_t* y,
                                    void* stream);

/* MXFP4 x MXFP4 GEMM on gfx950's block-scaled MFMA (the matrix cores take
 * the E2M1 codes and E8M0 bytes as stored):
 *   C[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k]        (TN, K-major)
 * with exact products and fp32 accumulation.  a_q [M][K/2], a_sf [M][K/32],
 * b_q [N][K/2], b_sf [N][K/32]; c [M][N] float, fully written (zeros when
 * K == 0).
 * Errors: EINVAL (K % 32 != 0, K > 2^23, M above 65535 * 256, null
 *   pointers), EALIGN (a_q, b_q, c not 16-byte aligned), ENOTSUP, EHIP. */
nvfp4_status nvfp4_mxfp4_gemm(const uint8_t* a_q, const uint8_t* a_sf, const uint8_t* b_q, const uint8_t* b_sf,
                              int64_t M, int64_t N, int64_t K, float* c, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
