/*
 * NVFP4 two-level microscaling -- CPU ORACLE (test infrastructure only).
 *
 * This file is the slow, plain reference that the HIP library is checked
 * against.  Only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load it; the product library never links or calls it, and
 * the two share no code, headers, tables or constants.
 *
 * What it computes, and where the pages fix it:
 *  - E2M1 element values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}: 1 sign, 2 exponent,
 *    1 mantissa bit (axbrief.com, "NVFP4: how NVIDIA pre-trained a 12B model
 *    on 10 trillion tokens", section "E2M1 format and two-level scaling";
 *    iwan.kr, "NVIDIA shrank GLM-5.2 to 4 bits", section 3 "Terminology:
 *    quantization and NVFP4", which counts 15 distinct values).
 *  - 16-element blocks sharing one E4M3 scale, plus one FP32 scale per tensor
 *    (same two sections; theddari.com, "What is FP4 quantization? KV cache in
 *    4 bits", format-comparison table).
 *  - The tensor-level FP32 scale sets the overall range and the block scale
 *    maps each block's amax close to the FP4 maximum (axbrief.com, section
 *    "E2M1 format and two-level scaling").
 * Where the pages are silent the recipe is the plainest reading:
 *  g  = RN32(amax / (6*448))           (448 = E4M3 maximum, 6 = E2M1 maximum)
 *  d6 = RN32(6*g)
 *  s  = E4M3_RNE_SAT(RN32(block_amax / d6))     (0 when d6 == 0)
 *  d  = RN32(s*g)
 *  code = sign(x)<<3 | E2M1_RNE_SAT(RN32(|x| / d))   (signed zero when d == 0)
 *  byte j of a row = code[2j] | code[2j+1] << 4
 *  dequant: bf16_RNE(RN32((E2M1(code)*s) * g)), sign from code bit 3
 * Every RN32 step is ONE IEEE-754 binary32 operation, round-to-nearest-even.
 * Build with -O2 -ffp-contract=off, no fast-math, no FTZ/DAZ (x86-64 SSE
 * float arithmetic is then exactly binary32 with one rounding per operation).
 * Rounding onto the E2M1 and E4M3 grids is done by brute-force nearest search
 * with ties to the even code -- the definition, not a shortcut.
 * Inputs are required to be finite; non-finite inputs return an error.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------- scalar formats ---------- */

/* E2M1 magnitude for code bits 2..0 (exponent bias 1, one mantissa bit). */
static const double kE2M1Mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code) {
  double m = kE2M1Mag[code & 7];
  return (code & 8) ? -m : m;
}

/* Nearest E2M1 magnitude code for y >= 0, ties to the even code, saturating
 * at 6 (the representable range ends at +-6; +inf from an overflowed quotient
 * saturates too).  Returns -1 for NaN or negative input. */
int orc_e2m1_encode(float y) {
  if (!(y >= 0.0f)) return -1;
  if (y > 6.0f) return 7;
  int best = 0;
  double bestd = fabs((double)y - kE2M1Mag[0]);
  for (int k = 1; k < 8; ++k) {
    double d = fabs((double)y - kE2M1Mag[k]);
    if (d < bestd || (d == bestd && (k & 1) == 0)) { best = k; bestd = d; }
  }
  return best;
}

/* OCP E4M3FN value of a non-negative scale byte 0x00..0x7E:
 * normal (1+m/8)*2^(e-7), subnormal m*2^-9; 0x7F (NaN) is never produced. */
double orc_e4m3_value(int byte) {
  int e = (byte >> 3) & 15, m = byte & 7;
  if (e == 0) return ldexp((double)m, -9);
  return ldexp(1.0 + m / 8.0, e - 7);
}

/* Nearest E4M3 byte for v >= 0, ties to the even mantissa, saturating at 448
 * (+inf included).  Returns -1 for NaN or negative input. */
int orc_e4m3_encode(float v) {
  if (!(v >= 0.0f)) return -1;
  if (v >= 448.0f) return 0x7E;
  int best = 0;
  double bestd = fabs((double)v);
  for (int b = 1; b <= 0x7E; ++b) {
    double d = fabs((double)v - orc_e4m3_value(b));
    if (d < bestd || (d == bestd && (b & 1) == 0)) { best = b; bestd = d; }
  }
  return best;
}

float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* bf16 nearest to a finite f32, ties to even; overflow gives +-inf. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t lo = (uint16_t)(u >> 16);          /* toward zero */
  if (((uint32_t)lo << 16) == u) return lo;   /* exact */
  uint16_t hi = (uint16_t)(lo + 1);           /* next magnitude up */
  double a = fabs((double)f);
  double vlo = fabs((double)orc_bf16_to_f32(lo));
  double vhi = ((hi & 0x7F80) == 0x7F80) ? ldexp(1.0, 128) : fabs((double)orc_bf16_to_f32(hi));
  double dlo = a - vlo, dhi = vhi - a;
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo & 1) ? hi : lo;
}

static int bf16_is_finite(uint16_t h) { return (h & 0x7F80) != 0x7F80; }
static float bf16_abs(uint16_t h) { return fabsf(orc_bf16_to_f32(h)); }

/* ---------- the two-level scales ---------- */

/* Step 1-2: tensor amax and the FP32 tensor scale g = RN32(amax / 2688). */
float orc_global_scale(float amax) { return amax / 2688.0f; }

/* Step 3-4: block scale byte from block amax and g. */
int orc_block_scale(float bamax, float g) {
  float d6 = 6.0f * g;
  if (d6 == 0.0f) return 0;
  return orc_e4m3_encode(bamax / d6);
}

/* Step 5-6: one element's 4-bit code given g and its block's scale byte. */
int orc_encode_element(uint16_t x, float g, int sbyte) {
  int sign = (x >> 15) & 1;
  float s = (float)orc_e4m3_value(sbyte);
  float d = s * g;
  if (d == 0.0f) return sign << 3;
  float y = bf16_abs(x) / d;
  return (sign << 3) | orc_e2m1_encode(y);
}

/* Encode one row of `cols` values (cols % 16 == 0) with tensor scale g. */
static void encode_row(const uint16_t* x, int64_t cols, float g, uint8_t* q, uint8_t* sf) {
  for (int64_t b = 0; b < cols / 16; ++b) {
    const uint16_t* xb = x + 16 * b;
    float bamax = 0.0f;
    for (int i = 0; i < 16; ++i) bamax = fmaxf(bamax, bf16_abs(xb[i]));
    int sbyte = orc_block_scale(bamax, g);
    sf[b] = (uint8_t)sbyte;
    for (int i = 0; i < 16; i += 2) {
      int c0 = orc_encode_element(xb[i], g, sbyte);
      int c1 = orc_encode_element(xb[i + 1], g, sbyte);
      q[8 * b + i / 2] = (uint8_t)(c0 | (c1 << 4));   /* element 2j in the low nibble */
    }
  }
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Full quantize: x [batch][rows][cols] bf16 -> q [batch][rows][cols/2],
 * sf [batch][rows][cols/16], g [batch].  Returns 0, or -1 on bad shape or a
 * non-finite input. */
int orc_quantize(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                 uint8_t* q, uint8_t* sf, float* g, int nthreads) {
  if (batch < 0 || rows < 0 || cols < 0 || cols % 16) return -1;
  set_threads(nthreads);
  const int64_t n = rows * cols;
  for (int64_t t = 0; t < batch; ++t) {
    const uint16_t* xt = x + t * n;
    float amax = 0.0f;
    int bad = 0;
#pragma omp parallel for reduction(max : amax) reduction(| : bad)
    for (int64_t i = 0; i < n; ++i) {
      if (!bf16_is_finite(xt[i])) bad = 1;
      amax = fmaxf(amax, bf16_abs(xt[i]));
    }
    if (bad) return -1;
    float gt = orc_global_scale(amax);
    g[t] = gt;
#pragma omp parallel for
    for (int64_t r = 0; r < rows; ++r)
      encode_row(xt + r * cols, cols, gt, q + (t * rows + r) * (cols / 2), sf + (t * rows + r) * (cols / 16));
  }
  return 0;
}

/* Quantize with caller-supplied tensor scales g[batch] (no amax pass). */
int orc_quantize_with_scale(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                            const float* g, uint8_t* q, uint8_t* sf, int nthreads) {
  if (batch < 0 || rows < 0 || cols < 0 || cols % 16) return -1;
  set_threads(nthreads);
  const int64_t n = rows * cols;
  for (int64_t t = 0; t < batch; ++t) {
    if (!(g[t] >= 0.0f) || isinf(g[t])) return -1;
    int bad = 0;
#pragma omp parallel for reduction(| : bad)
    for (int64_t i = 0; i < n; ++i)
      if (!bf16_is_finite(x[t * n + i])) bad = 1;
    if (bad) return -1;
#pragma omp parallel for
    for (int64_t r = 0; r < rows; ++r)
      encode_row(x + t * n + r * cols, cols, g[t], q + (t * rows + r) * (cols / 2), sf + (t * rows + r) * (cols / 16));
  }
  return 0;
}

/* One element's decoded fp32 value: RN32((E2M1(code) * s) * g). */
float orc_decode_element(int code, int sbyte, float g) {
  float m = (float)kE2M1Mag[code & 7];
  float s = (float)orc_e4m3_value(sbyte);
  float v = (m * s) * g;      /* m*s is exact in fp32; one rounding for *g */
  return (code & 8) ? -v : v;
}

/* Dequantize to bf16: y [batch][rows][cols]. */
int orc_dequantize(const uint8_t* q, const uint8_t* sf, const float* g, int64_t batch, int64_t rows,
                   int64_t cols, uint16_t* y, int nthreads) {
  if (batch < 0 || rows < 0 || cols < 0 || cols % 16) return -1;
  set_threads(nthreads);
  for (int64_t t = 0; t < batch; ++t) {
    const float gt = g[t];
#pragma omp parallel for
    for (int64_t r = 0; r < rows; ++r) {
      const int64_t row = t * rows + r;
      for (int64_t c = 0; c < cols; ++c) {
        int byte = q[row * (cols / 2) + c / 2];
        int code = (c & 1) ? (byte >> 4) : (byte & 15);
        int sbyte = sf[row * (cols / 16) + c / 16];
        y[row * cols + c] = orc_f32_to_bf16(orc_decode_element(code, sbyte, gt));
      }
    }
  }
  return 0;
}

/* Exact fp64 value E2M1(code) * s of every element, WITHOUT the tensor
 * scale (the GEMM and decode-QK references apply g separately in fp64). */
int orc_dequantize_f64_unscaled(const uint8_t* q, const uint8_t* sf, int64_t rows, int64_t cols,
                                double* y, int nthreads) {
  if (rows < 0 || cols < 0 || cols % 16) return -1;
  set_threads(nthreads);
#pragma omp parallel for
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      int byte = q[r * (cols / 2) + c / 2];
      int code = (c & 1) ? (byte >> 4) : (byte & 15);
      y[r * cols + c] = orc_e2m1_value(code) * orc_e4m3_value(sf[r * (cols / 16) + c / 16]);
    }
  return 0;
}

/* Array helpers for the exhaustive self-tests. */
void orc_e2m1_encode_array(const float* y, int64_t n, int8_t* out, int nthreads) {
  set_threads(nthreads);
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) out[i] = (int8_t)orc_e2m1_encode(y[i]);
}

void orc_e4m3_encode_array(const float* v, int64_t n, int16_t* out, int nthreads) {
  set_threads(nthreads);
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) out[i] = (int16_t)orc_e4m3_encode(v[i]);
}

void orc_f32_to_bf16_array(const float* f, int64_t n, uint16_t* out, int nthreads) {
  set_threads(nthreads);
#pragma omp parallel for
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(f[i]);
}

/* ---------- MXFP4: 32-value blocks, power-of-two scale, no tensor scale ----------
 *
 * The earlier microscaling format shares one power-of-two (UE8M0) scale among
 * 32 E2M1 values, about 4.25 bits per value (iwan.kr, "NVIDIA shrank GLM-5.2
 * to 4 bits", section 3 "Terminology"; axbrief.com, "NVFP4: how NVIDIA
 * pre-trained a 12B model on 10 trillion tokens", sections "E2M1 format and
 * two-level scaling" and "36% token efficiency and Blackwell speed";
 * theddari.com, "What is FP4 quantization? KV cache in 4 bits", format
 * comparison table).  The pages do not say how the exponent is chosen; the
 * reading here is the published Microscaling (MX) definition of the format:
 *   X = floor(log2(block amax)) - 2     (2 = exponent of E2M1's largest value,
 *                                         6 = 1.5 * 2^2), clamped to [-127, 127];
 *                                        an all-zero block takes X = -127
 *   scale byte = X + 127                 (E8M0: value 2^(byte-127), 255 = NaN)
 *   code = sign(x)<<3 | E2M1_RNE_SAT(RN32(|x| / 2^X))
 *   dequant: bf16_RNE(RN32(E2M1(code) * 2^X))
 * Values between 6 * 2^X and 8 * 2^X saturate to 6 * 2^X.  Codes are packed
 * as for NVFP4 (element 2j in the low nibble of byte j). */

double orc_e8m0_value(int byte) { return byte == 255 ? NAN : ldexp(1.0, byte - 127); }

/* Scale byte of a block from its amax (>= 0, finite); -1 otherwise.  The
 * exponent floor(log2(bamax)) is found by search: the largest e with
 * 2^e <= bamax. */
int orc_mx_block_scale(float bamax) {
  if (!(bamax >= 0.0f) || isinf(bamax)) return -1;
  if (bamax == 0.0f) return 0;
  int e = -160;
  while (ldexp(1.0, e + 1) <= (double)bamax) ++e;
  int x = e - 2;
  if (x < -127) x = -127;
  if (x > 127) x = 127;
  return x + 127;
}

/* One element's code given its block's scale byte (0..254). */
int orc_mx_encode_element(uint16_t x, int sbyte) {
  int sign = (x >> 15) & 1;
  float sc = (float)orc_e8m0_value(sbyte);       /* exact: 2^-127 .. 2^127 */
  float y = bf16_abs(x) / sc;
  return (sign << 3) | orc_e2m1_encode(y);
}

/* One element's decoded fp32 value RN32(E2M1(code) * 2^X); NaN for byte 255. */
float orc_mx_decode_element(int code, int sbyte) {
  if (sbyte == 255) return NAN;
  float m = (float)kE2M1Mag[code & 7];
  float v = m * (float)orc_e8m0_value(sbyte);
  return (code & 8) ? -v : v;
}

/* x [rows][cols] bf16 (cols % 32 == 0) -> q [rows][cols/2], sf [rows][cols/32].
 * Returns 0, or -1 on a bad shape or a non-finite input. */
int orc_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* q, uint8_t* sf, int nthreads) {
  if (rows < 0 || cols < 0 || cols % 32) return -1;
  set_threads(nthreads);
  int bad = 0;
#pragma omp parallel for reduction(| : bad)
  for (int64_t i = 0; i < rows * cols; ++i)
    if (!bf16_is_finite(x[i])) bad = 1;
  if (bad) return -1;
#pragma omp parallel for
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < cols / 32; ++b) {
      const uint16_t* xb = x + r * cols + 32 * b;
      float bamax = 0.0f;
      for (int i = 0; i < 32; ++i) bamax = fmaxf(bamax, bf16_abs(xb[i]));
      int sbyte = orc_mx_block_scale(bamax);
      sf[r * (cols / 32) + b] = (uint8_t)sbyte;
      for (int i = 0; i < 32; i += 2) {
        int c0 = orc_mx_encode_element(xb[i], sbyte);
        int c1 = orc_mx_encode_element(xb[i + 1], sbyte);
        q[r * (cols / 2) + 16 * b + i / 2] = (uint8_t)(c0 | (c1 << 4));
      }
    }
  return 0;
}

/* q [rows][cols/2], sf [rows][cols/32] -> y [rows][cols] bf16. */
int orc_mx_dequantize(const uint8_t* q, const uint8_t* sf, int64_t rows, int64_t cols, uint16_t* y, int nthreads) {
  if (rows < 0 || cols < 0 || cols % 32) return -1;
  set_threads(nthreads);
#pragma omp parallel for
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      int byte = q[r * (cols / 2) + c / 2];
      int code = (c & 1) ? (byte >> 4) : (byte & 15);
      y[r * cols + c] = orc_f32_to_bf16(orc_mx_decode_element(code, sf[r * (cols / 32) + c / 32]));
    }
  return 0;
}

/* Exact fp64 value E2M1(code) * 2^X of every element (NaN for byte 255). */
int orc_mx_dequantize_f64(const uint8_t* q, const uint8_t* sf, int64_t rows, int64_t cols, double* y,
                          int nthreads) {
  if (rows < 0 || cols < 0 || cols % 32) return -1;
  set_threads(nthreads);
#pragma omp parallel for
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) {
      int byte = q[r * (cols / 2) + c / 2];
      int code = (c & 1) ? (byte >> 4) : (byte & 15);
      y[r * cols + c] = orc_e2m1_value(code) * orc_e8m0_value(sf[r * (cols / 32) + c / 32]);
    }
  return 0;
}

/* ---------- training-recipe variants ----------
 *
 * The pages' training recipe (axbrief.com, "NVFP4: how NVIDIA pre-trained a
 * 12B model on 10 trillion tokens", section "Four stabilizers for training:
 * from RHT to stochastic rounding") quantizes the operands of the Fprop,
 * Dgrad and Wgrad GEMMs and adds:
 *  - 16x16 2D block scaling of weights, so a weight and its transpose have
 *    the same quantized form;
 *  - a random Hadamard transform of the Wgrad inputs: a 16x16 Hadamard
 *    matrix times a random +-1 sign vector;
 *  - stochastic rounding of gradients: a value between two neighbours
 *    rounds up with probability equal to its distance from the lower one
 *    over the gap (0.7 between 0 and 1 becomes 1 with probability 0.7).
 * Readings where the pages are silent:
 *  - COLWISE quantizes x^T (blocks run down the columns of x): the Dgrad /
 *    Wgrad operand layout, whose contraction runs over x's rows.
 *  - 2D: one E4M3 scale per 16x16 tile from the tile's amax; the byte is
 *    stored for each of the tile's 16 rows in the usual [rows][cols/16]
 *    layout, so every NVFP4 consumer reads it unchanged.
 *  - RHT acts on each 16-value block along the block direction:
 *    v = H16 (s .* x) / 4, H16 the Sylvester Hadamard matrix
 *    (H[i][j] = (-1)^popcount(i & j)) and s the caller's signs (bit j of a
 *    16-bit mask set means s_j = -1).  It is computed in fp32 as the fast
 *    Walsh-Hadamard transform: stages h = 1, 2, 4, 8, each replacing the
 *    pair (v[i], v[i+h]) (i & h == 0) by (v[i] + v[i+h], v[i] - v[i+h]),
 *    then a multiply by 1/4.  The quantizer takes those fp32 values (the
 *    recipe's amax, quotients and codes run on them unchanged).
 *  - SR replaces only the element rounding E2M1_RNE_SAT(y): with lo the
 *    largest E2M1 magnitude <= y and hi the next (y >= 6 gives 6), the code
 *    rounds up when u < (y - lo) / (hi - lo), u a 16-bit uniform draw u16 /
 *    65536.  Scales stay round-to-nearest.
 *  - The draws come from Philox4x32-10 (Salmon et al., "Parallel random
 *    numbers: as easy as 1, 2, 3", SC 2011): for the element at linear
 *    index i of the output code array, counter (n mod 2^32, n >> 32, 0, 0)
 *    with n = i / 8 + offset, key (seed mod 2^32, seed >> 32); the element
 *    takes 16-bit half (i mod 2) of output word (i mod 8) / 2.
 */

#define ORC_COLWISE 1u
#define ORC_2D 2u
#define ORC_RHT 4u
#define ORC_SR 8u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;                 /* Weyl key schedule */
      k1 += 0xBB67AE85u;
    }
    uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* 16-bit draw of the element at output index i. */
static uint32_t sr_draw(int64_t i, uint64_t seed, uint64_t offset) {
  uint64_t n = (uint64_t)i / 8 + offset;
  uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return (out[(i & 7) >> 1] >> (16 * (i & 1))) & 0xFFFFu;
}

/* Stochastic E2M1 magnitude code of y >= 0 with the 16-bit draw u16. */
int orc_e2m1_encode_sr(float y, uint32_t u16) {
  if (!(y >= 0.0f)) return -1;
  if (y >= 6.0f) return 7;
  int lo = 0;
  while (lo < 7 && kE2M1Mag[lo + 1] <= (double)y) ++lo;
  double p = ((double)y - kE2M1Mag[lo]) / (kE2M1Mag[lo + 1] - kE2M1Mag[lo]);   /* exact */
  return (double)u16 / 65536.0 < p ? lo + 1 : lo;
}

/* In-place RHT of one 16-value block (fp32, the stage order above). */
void orc_rht16(float v[16], uint32_t signs) {
  for (int j = 0; j < 16; ++j)
    if ((signs >> j) & 1u) v[j] = -v[j];
  for (int h = 1; h < 16; h <<= 1)
    for (int i = 0; i < 16; ++i)
      if ((i & h) == 0) {
        float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
  for (int j = 0; j < 16; ++j) v[j] = v[j] * 0.25f;
}

/* Element code from an fp32 value (the variant path: the value may be an
 * RHT output), given d = RN32(s g) of its block. */
static int encode_value(float v, float d, int sr, uint32_t u16) {
  int sign = signbit(v) ? 1 : 0;
  if (d == 0.0f) return sign << 3;
  float y = fabsf(v) / d;
  return (sign << 3) | (sr ? orc_e2m1_encode_sr(y, u16) : orc_e2m1_encode(y));
}

/* Variant quantize: x [batch][rows][cols] bf16 -> q, sf, g.  Output matrix
 * per tensor is [R][C] = [rows][cols], or [cols][rows] with COLWISE:
 * q [batch][R][C/2], sf [batch][R][C/16], g [batch].  Requires cols % 16 ==
 * 0, and rows % 16 == 0 with COLWISE or 2D; 2D with RHT is not a variant
 * (-2).  Returns 0, -1 on bad shapes / non-finite input. */
int orc_quantize_ex(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, uint32_t variant,
                    uint32_t signs, uint64_t seed, uint64_t offset, uint8_t* q, uint8_t* sf, float* g) {
  const int colwise = (variant & ORC_COLWISE) != 0, two_d = (variant & ORC_2D) != 0;
  const int rht = (variant & ORC_RHT) != 0, sr = (variant & ORC_SR) != 0;
  if (batch < 0 || rows < 0 || cols < 0 || cols % 16) return -1;
  if ((colwise || two_d) && rows % 16) return -1;
  if (two_d && rht) return -2;
  const int64_t R = colwise ? cols : rows, C = colwise ? rows : cols;
  const int64_t n = rows * cols;
  float* v = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  if (!v) return -1;
  for (int64_t t = 0; t < batch; ++t) {
    const uint16_t* xt = x + t * n;
    /* the output-oriented values v[r][c] (x or x^T), RHT per block */
    for (int64_t r = 0; r < R; ++r)
      for (int64_t c = 0; c < C; ++c) {
        uint16_t b = colwise ? xt[c * cols + r] : xt[r * cols + c];
        if (!bf16_is_finite(b)) { free(v); return -1; }
        v[r * C + c] = orc_bf16_to_f32(b);
      }
    if (rht)
      for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; c += 16) orc_rht16(v + r * C + c, signs);
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float gt = orc_global_scale(amax);
    g[t] = gt;
    for (int64_t r = 0; r < R; ++r)
      for (int64_t b = 0; b < C / 16; ++b) {
        float bamax = 0.0f;
        if (two_d) {                                   /* the 16x16 tile holding (r, b) */
          int64_t r0 = r - r % 16;
          for (int64_t rr = r0; rr < r0 + 16; ++rr)
            for (int i = 0; i < 16; ++i) bamax = fmaxf(bamax, fabsf(v[rr * C + 16 * b + i]));
        } else {
          for (int i = 0; i < 16; ++i) bamax = fmaxf(bamax, fabsf(v[r * C + 16 * b + i]));
        }
        const int sbyte = orc_block_scale(bamax, gt);
        sf[(t * R + r) * (C / 16) + b] = (uint8_t)sbyte;
        const float d = (float)orc_e4m3_value(sbyte) * gt;
        for (int i = 0; i < 16; i += 2) {
          const int64_t i0 = (t * R + r) * C + 16 * b + i;          /* output linear index */
          int c0 = encode_value(v[r * C + 16 * b + i], d, sr, sr ? sr_draw(i0, seed, offset) : 0u);
          int c1 = encode_value(v[r * C + 16 * b + i + 1], d, sr, sr ? sr_draw(i0 + 1, seed, offset) : 0u);
          q[i0 / 2] = (uint8_t)(c0 | (c1 << 4));
        }
      }
  }
  free(v);
  return 0;
}
