/*
 * nm_oracle.c -- CPU oracle (test infrastructure only; see nm_oracle.h).
 *
 * Plain, slow and deliberately literal.  Every step follows a definition
 * stated on the source pages; where the pages leave a step open the reading
 * is named at that step.
 */
#include "nm_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Exact magnitudes.                                                         */
/*                                                                           */
/* ASP's mn_1d_best ([SRSTE] "NVIDA Apex内的静态掩码稀疏") scores a pattern by the */
/* sum of |w| over the kept positions.  A floating-point sum can round two    */
/* different scores to the same number, so the oracle sums exactly: every     */
/* finite float of a binary format is an integer multiple of that format's   */
/* smallest subnormal, and that integer is                                   */
/*     e == 0 :  f                      (subnormal or zero)                   */
/*     e >  0 :  (2^p + f) << (e - 1)   (normal)                              */
/* for exponent field e and p-bit fraction field f.  The same formula applied */
/* to the all-ones exponent gives Inf/NaN an integer larger than every finite */
/* value, which is the order of the sign-cleared bit pattern.                */
/* fp32 needs up to 2^24 << 254 < 2^278; five 64-bit limbs hold sums of up to */
/* 2^42 such terms, far more than any group.                                  */
/* ------------------------------------------------------------------------ */

#define LIMBS 5
typedef struct {
  uint64_t w[LIMBS]; /* little-endian limbs */
} big_t;

static void big_zero(big_t* a) { memset(a, 0, sizeof(*a)); }

static void big_add(big_t* acc, const big_t* x) {
  uint64_t carry = 0;
  for (int i = 0; i < LIMBS; i++) {
    uint64_t s = acc->w[i] + x->w[i];
    uint64_t c1 = s < acc->w[i];
    uint64_t s2 = s + carry;
    uint64_t c2 = s2 < s;
    acc->w[i] = s2;
    carry = c1 | c2;
  }
}

/* -1, 0, +1 as a <, ==, > b */
static int big_cmp(const big_t* a, const big_t* b) {
  for (int i = LIMBS - 1; i >= 0; i--) {
    if (a->w[i] < b->w[i]) return -1;
    if (a->w[i] > b->w[i]) return 1;
  }
  return 0;
}

/* value << shift into a big_t; value < 2^25, shift < 256 */
static void big_from_shifted(big_t* out, uint64_t value, int shift) {
  big_zero(out);
  int limb = shift / 64, off = shift % 64;
  out->w[limb] = value << off;
  if (off != 0 && limb + 1 < LIMBS) out->w[limb + 1] = value >> (64 - off);
}

static uint32_t raw_bits(const void* p, int dt, int64_t i) {
  if (dt == NMO_F32) return ((const uint32_t*)p)[i];
  if (dt == NMO_I8 || dt == NMO_FP8) return ((const uint8_t*)p)[i];
  return ((const uint16_t*)p)[i];
}

static int elem_size(int dt) { return dt == NMO_F32 ? 4 : (dt == NMO_I8 || dt == NMO_FP8) ? 1 : 2; }

/* exact |w| of element i, as an integer multiple of the smallest subnormal (of 1 for int8) */
static void exact_magnitude(const void* W, int dt, int64_t i, big_t* out) {
  uint32_t bits = raw_bits(W, dt, i);
  uint32_t e, f;
  int p;
  if (dt == NMO_I8) { /* two's complement: |-128| = 128 */
    int v = (int)(int8_t)(uint8_t)bits;
    big_from_shifted(out, (uint64_t)(v < 0 ? -v : v), 0);
    return;
  }
  if (dt == NMO_F32) {
    e = (bits >> 23) & 0xFFu;
    f = bits & 0x7FFFFFu;
    p = 23;
  } else if (dt == NMO_FP8) { /* OCP E4M3: 1 sign, 4 exponent, 3 fraction bits */
    e = (bits >> 3) & 0xFu;
    f = bits & 0x7u;
    p = 3;
  } else if (dt == NMO_BF16) { /* bf16 = upper half of an fp32 */
    e = (bits >> 7) & 0xFFu;
    f = (bits & 0x7Fu) << 16;
    p = 23;
  } else { /* fp16 */
    e = (bits >> 10) & 0x1Fu;
    f = bits & 0x3FFu;
    p = 10;
  }
  if (e == 0)
    big_from_shifted(out, f, 0);
  else
    big_from_shifted(out, ((uint64_t)1 << p) + f, (int)e - 1);
}

double nmo_to_double(const void* p, int dt, int64_t i) {
  uint32_t bits = raw_bits(p, dt, i);
  if (dt == NMO_I8) return (double)(int8_t)(uint8_t)bits;
  if (dt == NMO_FP8) {
    /* OCP FP8 E4M3 (bias 7): no infinities; exponent 15 with fraction 7 is NaN */
    int s8 = (bits >> 7) & 1, e8 = (bits >> 3) & 0xF, f8 = bits & 7;
    double v8;
    if (e8 == 0)
      v8 = ldexp((double)f8, -9);
    else if (e8 == 15 && f8 == 7)
      v8 = NAN;
    else
      v8 = ldexp((double)(8 + f8), e8 - 10);
    return s8 ? -v8 : v8;
  }
  if (dt == NMO_F32) {
    float v;
    memcpy(&v, &bits, 4);
    return (double)v;
  }
  if (dt == NMO_BF16) {
    uint32_t b32 = bits << 16;
    float v;
    memcpy(&v, &b32, 4);
    return (double)v;
  }
  /* fp16: 1 sign, 5 exponent (bias 15), 10 fraction bits */
  int s = (bits >> 15) & 1;
  int e = (bits >> 10) & 0x1F;
  int f = bits & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return s ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Argument checks and metadata geometry                                     */
/* ------------------------------------------------------------------------ */

int nmo_meta_bits(int m) {
  switch (m) {
    case 2: return 1;
    case 4: return 2;
    case 8: return 3;
    case 16: return 4;
    default: return -1;
  }
}

int64_t nmo_meta_words_per_row(int64_t K, int n, int m) {
  int b = nmo_meta_bits(m);
  if (b < 0 || n < 1 || n > m || K < 0 || K % m != 0) return -1;
  int64_t bits = (K / m) * n * b;
  return (bits + 31) / 32;
}

static int check_args(int dt, int64_t R, int64_t K, int n, int m) {
  if (dt != NMO_F32 && dt != NMO_F16 && dt != NMO_BF16 && dt != NMO_I8 && dt != NMO_FP8)
    return -1;
  if (R < 0 || K < 0) return -2;
  if (nmo_meta_bits(m) < 0 || n < 1 || n > m) return -3;
  if (K % m != 0) return -4;
  return 0;
}

static void put_field(uint32_t* row, int64_t field, int b, uint32_t v) {
  int64_t bit = field * b;
  int64_t w = bit / 32;
  int off = (int)(bit % 32);
  row[w] |= (uint32_t)((uint64_t)v << off);
  if (off + b > 32) row[w + 1] |= v >> (32 - off);
}

static uint32_t get_field(const uint32_t* row, int64_t field, int b) {
  int64_t bit = field * b;
  int64_t w = bit / 32;
  int off = (int)(bit % 32);
  uint64_t window = row[w] >> off;
  if (off + b > 32) window |= (uint64_t)row[w + 1] << (32 - off);
  return (uint32_t)(window & ((1u << b) - 1u));
}

/* ------------------------------------------------------------------------ */
/* Group selection: ASP's exhaustive search ([SRSTE] "NVIDA Apex内的静态掩码稀疏"). */
/* Enumerate every set of n positions out of m (all valid N:M patterns) in   */
/* lexicographic order of the ascending index tuple, score each by the exact */
/* sum of the kept magnitudes, and keep the first pattern with the largest   */
/* score (a later pattern replaces it only when strictly larger).            */
/* ------------------------------------------------------------------------ */
static void best_pattern(const void* W, int dt, int64_t base, int n, int m, int* kept) {
  int idx[16];
  big_t mag[16], best, score;
  for (int i = 0; i < m; i++) exact_magnitude(W, dt, base + i, &mag[i]);
  for (int j = 0; j < n; j++) idx[j] = j;
  int have_best = 0;
  for (;;) {
    big_zero(&score);
    for (int j = 0; j < n; j++) big_add(&score, &mag[idx[j]]);
    if (!have_best || big_cmp(&score, &best) > 0) {
      best = score;
      for (int j = 0; j < n; j++) kept[j] = idx[j];
      have_best = 1;
    }
    /* next combination in lexicographic order */
    int j = n - 1;
    while (j >= 0 && idx[j] == m - n + j) j--;
    if (j < 0) break;
    idx[j]++;
    for (int k = j + 1; k < n; k++) idx[k] = idx[k - 1] + 1;
  }
}

int nmo_mask(const void* W, int dt, int64_t R, int64_t K, int n, int m, uint8_t* mask) {
  int rc = check_args(dt, R, K, n, m);
  if (rc) return rc;
  int kept[16];
  for (int64_t r = 0; r < R; r++) {
    for (int64_t g = 0; g < K / m; g++) {
      int64_t base = r * K + g * m;
      best_pattern(W, dt, base, n, m, kept);
      for (int i = 0; i < m; i++) mask[base + i] = 0;
      for (int j = 0; j < n; j++) mask[base + kept[j]] = 1;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Compression ([ASDNN] "2:4 Sparsity의 benefits"): the kept values of each   */
/* group, in ascending position order, form the value array (K*n/m per row,  */
/* always n per group even if the group holds more zeros); each kept value's */
/* position inside its group is written as a b-bit metadata field.           */
/* ------------------------------------------------------------------------ */
int nmo_compress(const void* W, int dt, int64_t R, int64_t K, int n, int m, void* values,
                 uint32_t* meta) {
  int rc = check_args(dt, R, K, n, m);
  if (rc) return rc;
  int b = nmo_meta_bits(m);
  int64_t wpr = nmo_meta_words_per_row(K, n, m);
  int64_t kv = K / m * n; /* values per row */
  int kept[16];
  for (int64_t r = 0; r < R; r++) {
    uint32_t* mrow = meta + r * wpr;
    for (int64_t w = 0; w < wpr; w++) mrow[w] = 0;
    for (int64_t g = 0; g < K / m; g++) {
      int64_t base = r * K + g * m;
      best_pattern(W, dt, base, n, m, kept);
      for (int j = 0; j < n; j++) {
        int64_t dst = r * kv + g * n + j;
        if (dt == NMO_F32)
          ((uint32_t*)values)[dst] = ((const uint32_t*)W)[base + kept[j]];
        else if (dt == NMO_I8 || dt == NMO_FP8)
          ((uint8_t*)values)[dst] = ((const uint8_t*)W)[base + kept[j]];
        else
          ((uint16_t*)values)[dst] = ((const uint16_t*)W)[base + kept[j]];
        put_field(mrow, g * n + j, b, (uint32_t)kept[j]);
      }
    }
  }
  return 0;
}

/* Decompression: stored values back at their recorded positions, +0 elsewhere. */
int nmo_decompress(const void* values, const uint32_t* meta, int dt, int64_t R, int64_t K, int n,
                   int m, void* W_out) {
  int rc = check_args(dt, R, K, n, m);
  if (rc) return rc;
  int b = nmo_meta_bits(m);
  int64_t wpr = nmo_meta_words_per_row(K, n, m);
  int64_t kv = K / m * n;
  int s = elem_size(dt);
  memset(W_out, 0, (size_t)(R * K * s));
  for (int64_t r = 0; r < R; r++) {
    const uint32_t* mrow = meta + r * wpr;
    for (int64_t g = 0; g < K / m; g++) {
      for (int j = 0; j < n; j++) {
        int64_t pos = r * K + g * m + get_field(mrow, g * n + j, b);
        int64_t src = r * kv + g * n + j;
        if (dt == NMO_F32)
          ((uint32_t*)W_out)[pos] = ((const uint32_t*)values)[src];
        else if (dt == NMO_I8 || dt == NMO_FP8)
          ((uint8_t*)W_out)[pos] = ((const uint8_t*)values)[src];
        else
          ((uint16_t*)W_out)[pos] = ((const uint16_t*)values)[src];
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Sparse x dense product ([ASDNN] "Tensor Scores 상에서 구조적인 sparse GEMM"): */
/* the result is the ordinary dense product of the decompressed first operand */
/* with the dense second operand.  Inputs are converted to double exactly;   */
/* every product of two 16-bit or two fp32 inputs is exact in double, and the */
/* sum runs over ascending k.                                                */
/* ------------------------------------------------------------------------ */
static void decompress_row_double(const void* values, const uint32_t* meta, int dt, int64_t r,
                                  int64_t K, int n, int m, double* wd) {
  int b = nmo_meta_bits(m);
  int64_t wpr = nmo_meta_words_per_row(K, n, m);
  int64_t kv = K / m * n;
  const uint32_t* mrow = meta + r * wpr;
  for (int64_t k = 0; k < K; k++) wd[k] = 0.0;
  for (int64_t g = 0; g < K / m; g++)
    for (int j = 0; j < n; j++)
      wd[g * m + get_field(mrow, g * n + j, b)] = nmo_to_double(values, dt, r * kv + g * n + j);
}

int nmo_spmm_rows(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n, int m,
                  const void* X, int64_t T, int dt, int64_t r0, int64_t r1, double* Y) {
  int rc = check_args(dt, R, K, n, m);
  if (rc) return rc;
  if (T < 0 || r0 < 0 || r1 > R || r0 > r1) return -2;
  double* wd = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  double* xrow = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
  if (!wd || !xrow) {
    free(wd);
    free(xrow);
    return -5;
  }
  for (int64_t r = r0; r < r1; r++) {
    double* y = Y + r * T;
    for (int64_t t = 0; t < T; t++) y[t] = 0.0;
    decompress_row_double(values, meta, dt, r, K, n, m, wd);
    for (int64_t k = 0; k < K; k++) {
      for (int64_t t = 0; t < T; t++) xrow[t] = nmo_to_double(X, dt, k * T + t);
      for (int64_t t = 0; t < T; t++) y[t] += wd[k] * xrow[t];
    }
  }
  free(wd);
  free(xrow);
  return 0;
}

int nmo_spmm(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n, int m,
             const void* X, int64_t T, int dt, double* Y) {
  return nmo_spmm_rows(values, meta, R, K, n, m, X, T, dt, 0, R, Y);
}

int nmo_spmm_sample(const void* values, const uint32_t* meta, int64_t R, int64_t K, int n, int m,
                    const void* X, int64_t T, int dt, const int64_t* rs, const int64_t* ts,
                    int64_t count, double* out) {
  int rc = check_args(dt, R, K, n, m);
  if (rc) return rc;
  double* wd = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
  if (!wd) return -5;
  for (int64_t i = 0; i < count; i++) {
    int64_t r = rs[i], t = ts[i];
    if (r < 0 || r >= R || t < 0 || t >= T) {
      free(wd);
      return -2;
    }
    decompress_row_double(values, meta, dt, r, K, n, m, wd);
    double acc = 0.0;
    for (int64_t k = 0; k < K; k++) acc += wd[k] * nmo_to_double(X, dt, k * T + t);
    out[i] = acc;
  }
  free(wd);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* SR-STE ([SRSTE] "基于直通估计的动态掩码精炼化稀疏(SR-STE)").                */
/*                                                                           */
/* Forward: the mask is searched again from the current weights at every    */
/* step and the layer uses the weights times that mask.  Backward: the      */
/* gradient passes straight through where the mask keeps the weight and     */
/* gains decay * weight where it prunes it.                                  */
/* ------------------------------------------------------------------------ */

/* exact value of element i as a float (every fp16 and bf16 value is an fp32 value) */
static float elem_to_float(const void* p, int dt, int64_t i) {
  uint32_t bits = raw_bits(p, dt, i);
  float v;
  if (dt == NMO_F32) {
    memcpy(&v, &bits, 4);
    return v;
  }
  if (dt == NMO_BF16) {
    uint32_t b32 = bits << 16;
    memcpy(&v, &b32, 4);
    return v;
  }
  return (float)nmo_to_double(p, dt, i);
}

/* Round a float to the nearest bf16, ties to even.  bf16 is the upper half of   */
/* the fp32 encoding (same sign, exponent and leading 7 fraction bits), so the   */
/* discarded low 16 bits decide: above half an ulp rounds up, exactly half rounds */
/* to the even neighbour; a carry into the exponent (or into Inf) is the correct */
/* next value.  NaN stays NaN (quiet bit set).                                   */
static uint16_t float_to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t keep = u >> 16, rest = u & 0xFFFFu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
  return (uint16_t)keep;
}

/* Round a float to the nearest IEEE binary16, ties to even: 1 sign, 5 exponent  */
/* (bias 15) and 10 fraction bits.  |x| is scaled (exactly, in double) to units  */
/* of its binade's quantum and rounded to an integer with rint (the default      */
/* rounding mode is to nearest, ties to even).  Magnitudes from 65520 (half way  */
/* between the largest finite value 65504 and 2^16) up become Inf.               */
static uint16_t float_to_f16(float x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  double a = fabs((double)x);
  if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  if (a < ldexp(1.0, -14)) { /* subnormal binade: quantum 2^-24 */
    double q = rint(ldexp(a, 24)); /* 0 .. 1024; 1024 is the smallest normal's code */
    return (uint16_t)(sign | (uint16_t)q);
  }
  int ex;
  frexp(a, &ex);                   /* a = f * 2^ex, 0.5 <= f < 1 */
  int E = ex - 1;                  /* 2^E <= a < 2^(E+1), -14 <= E <= 15 */
  double q = rint(ldexp(a, 10 - E)); /* 1024 .. 2048 */
  if (q == 2048.0) {
    q = 1024.0;
    E += 1;
  }
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0));
}

static void store_rounded(void* out, int dt, int64_t i, float v) {
  if (dt == NMO_F32)
    memcpy((uint32_t*)out + i, &v, 4);
  else if (dt == NMO_BF16)
    ((uint16_t*)out)[i] = float_to_bf16(v);
  else
    ((uint16_t*)out)[i] = float_to_f16(v);
}

int nmo_round_from_f32(const float* in, int dt, int64_t count, void* out) {
  if (dt != NMO_F32 && dt != NMO_F16 && dt != NMO_BF16) return -1;
  if (count < 0) return -2;
  for (int64_t i = 0; i < count; i++) store_rounded(out, dt, i, in[i]);
  return 0;
}

static void copy_elem(void* dst, const void* src, int dt, int64_t i) {
  if (dt == NMO_F32)
    ((uint32_t*)dst)[i] = ((const uint32_t*)src)[i];
  else
    ((uint16_t*)dst)[i] = ((const uint16_t*)src)[i];
}

static void zero_elem(void* dst, int dt, int64_t i) {
  if (dt == NMO_F32)
    ((uint32_t*)dst)[i] = 0u;
  else
    ((uint16_t*)dst)[i] = 0u;
}

/* Forward weight: kept elements unchanged (bit for bit), pruned ones +0. */
int nmo_prune(const void* W, int dt, int64_t R, int64_t K, int n, int m, void* W_out) {
  int rc = check_args(dt, R, K, n, m);
  if (rc) return rc;
  if (dt == NMO_I8 || dt == NMO_FP8) return -1; /* SR-STE trains 16/32-bit weights */
  int kept[16];
  for (int64_t r = 0; r < R; r++) {
    for (int64_t g = 0; g < K / m; g++) {
      int64_t base = r * K + g * m;
      best_pattern(W, dt, base, n, m, kept);
      for (int i = 0; i < m; i++) zero_elem(W_out, dt, base + i);
      for (int j = 0; j < n; j++) copy_elem(W_out, W, dt, base + kept[j]);
    }
  }
  return 0;
}

/* Backward: out = G where the weight is kept (bit for bit); where it is pruned,  */
/* out = G + decay * W evaluated as the printed backward does for a float32       */
/* decay: p = decay * w rounded to fp32, s = g + p rounded to fp32, then s       */
/* rounded once to dt.  The operands w and g are the exact fp32 values of the    */
/* stored elements.  Each operation is its own IEEE single operation (this file  */
/* is compiled with -ffp-contract=off, so no fused multiply-add).                */
int nmo_srste_grad(const void* W, const void* G, int dt, int64_t R, int64_t K, int n, int m,
                   float decay, void* G_out) {
  int rc = check_args(dt, R, K, n, m);
  if (rc) return rc;
  if (dt == NMO_I8 || dt == NMO_FP8) return -1;
  int kept[16];
  for (int64_t r = 0; r < R; r++) {
    for (int64_t g = 0; g < K / m; g++) {
      int64_t base = r * K + g * m;
      int is_kept[16] = {0};
      best_pattern(W, dt, base, n, m, kept);
      for (int j = 0; j < n; j++) is_kept[kept[j]] = 1;
      for (int i = 0; i < m; i++) {
        if (is_kept[i]) {
          copy_elem(G_out, G, dt, base + i);
        } else {
          float w = elem_to_float(W, dt, base + i);
          float gr = elem_to_float(G, dt, base + i);
          float p = decay * w;
          float s = gr + p;
          store_rounded(G_out, dt, base + i, s);
        }
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Transposable N:M masks ([TRANS] "提出的方法").                              */
/*                                                                           */
/* W is cut into m x m blocks (rows and columns aligned at multiples of m).  */
/* A transposable mask keeps at most n entries in every row and every column */
/* of every block, so both W and its transpose are N:M along their           */
/* contiguous dimension and one mask serves the forward and the backward    */
/* product.  The best such mask maximises the kept L1 norm of each block (a  */
/* minimum-cost flow problem); the fast method is a greedy 2-approximation.  */
/* ------------------------------------------------------------------------ */

static int check_tshape(int dt, int64_t R, int64_t K, int n, int m) {
  int rc = check_args(dt, R, K, n, m);
  if (rc) return rc;
  if (dt == NMO_I8 || dt == NMO_FP8) return -1; /* built for trained 16/32-bit weights */
  if (R % m != 0) return -4;
  return 0;
}

/* Greedy: take the block's entries in descending exact magnitude (equal     */
/* magnitudes in ascending row-major position inside the block) and keep an  */
/* entry whenever its row and its column still hold fewer than n kept ones.  */
static void greedy_block(const void* W, int dt, int64_t K, int64_t r0, int64_t c0, int n, int m,
                         uint8_t* keep /* m*m, row-major */) {
  int order[256];
  big_t mag[256];
  int cnt = m * m;
  for (int e = 0; e < cnt; e++) {
    exact_magnitude(W, dt, (r0 + e / m) * K + c0 + e % m, &mag[e]);
    order[e] = e;
  }
  /* insertion sort: larger magnitude first, lower position first on ties (stable) */
  for (int i = 1; i < cnt; i++) {
    int e = order[i], j = i - 1;
    while (j >= 0 && big_cmp(&mag[order[j]], &mag[e]) < 0) {
      order[j + 1] = order[j];
      j--;
    }
    order[j + 1] = e;
  }
  int rows[16] = {0}, cols[16] = {0};
  for (int e = 0; e < cnt; e++) keep[e] = 0;
  for (int i = 0; i < cnt; i++) {
    int e = order[i], r = e / m, c = e % m;
    if (rows[r] < n && cols[c] < n) {
      keep[e] = 1;
      rows[r]++;
      cols[c]++;
    }
  }
}

int nmo_tmask_greedy(const void* W, int dt, int64_t R, int64_t K, int n, int m, uint8_t* mask) {
  int rc = check_tshape(dt, R, K, n, m);
  if (rc) return rc;
  uint8_t keep[256];
  for (int64_t r0 = 0; r0 < R; r0 += m)
    for (int64_t c0 = 0; c0 < K; c0 += m) {
      greedy_block(W, dt, K, r0, c0, n, m, keep);
      for (int e = 0; e < m * m; e++) mask[(r0 + e / m) * K + c0 + e % m] = keep[e];
    }
  return 0;
}

/* The optimum, as a minimum-cost flow: source -> row i (capacity n), row i ->  */
/* column j (capacity 1, cost -|w_ij|), column j -> sink (capacity n).  Flow is */
/* pushed one unit at a time along a cheapest source-sink path of the residual  */
/* graph (Bellman-Ford, since costs are negative), while such a path lowers the */
/* cost; the row->column arcs that carry flow form the mask.  Costs are doubles */
/* (|w| of every format is exact in double); the optimum's ties are not fixed.  */
#define TF_MAXV (2 * 16 + 2)
int nmo_tmask_optimal(const void* W, int dt, int64_t R, int64_t K, int n, int m, uint8_t* mask,
                      double* kept_l1) {
  int rc = check_tshape(dt, R, K, n, m);
  if (rc) return rc;
  const int V = 2 * m + 2, S = 2 * m, T = 2 * m + 1;
  double total = 0.0;
  for (int64_t r0 = 0; r0 < R; r0 += m)
    for (int64_t c0 = 0; c0 < K; c0 += m) {
      double cost[TF_MAXV][TF_MAXV];
      int cap[TF_MAXV][TF_MAXV];
      for (int a = 0; a < V; a++)
        for (int b = 0; b < V; b++) {
          cost[a][b] = 0.0;
          cap[a][b] = 0;
        }
      for (int i = 0; i < m; i++) {
        cap[S][i] = n;
        cap[m + i][T] = n;
        for (int j = 0; j < m; j++) {
          double a = fabs(nmo_to_double(W, dt, (r0 + i) * K + c0 + j));
          if (isnan(a)) a = INFINITY;
          if (isinf(a)) a = 1e300; /* Inf and NaN outrank every finite value */
          cap[i][m + j] = 1;
          cost[i][m + j] = -a;
          cost[m + j][i] = a; /* residual arc */
        }
      }
      for (;;) {
        double dist[TF_MAXV];
        int prev[TF_MAXV];
        for (int v = 0; v < V; v++) {
          dist[v] = INFINITY;
          prev[v] = -1;
        }
        dist[S] = 0.0;
        for (int it = 0; it < V; it++) {
          int changed = 0;
          for (int a = 0; a < V; a++) {
            if (dist[a] == INFINITY) continue;
            for (int b = 0; b < V; b++)
              if (cap[a][b] > 0 && dist[a] + cost[a][b] < dist[b]) {
                dist[b] = dist[a] + cost[a][b];
                prev[b] = a;
                changed = 1;
              }
          }
          if (!changed) break;
        }
        if (dist[T] == INFINITY || dist[T] >= 0.0) break; /* no improving path left */
        for (int v = T; v != S; v = prev[v]) {
          cap[prev[v]][v] -= 1;
          cap[v][prev[v]] += 1;
        }
      }
      for (int i = 0; i < m; i++)
        for (int j = 0; j < m; j++) {
          int used = cap[i][m + j] == 0;
          mask[(r0 + i) * K + c0 + j] = (uint8_t)used;
          if (used) total += -cost[i][m + j];
        }
    }
  if (kept_l1) *kept_l1 = total;
  return 0;
}

/* Forward weight under the greedy transposable mask: W where kept, +0 where pruned. */
int nmo_tprune(const void* W, int dt, int64_t R, int64_t K, int n, int m, void* W_out) {
  int rc = check_tshape(dt, R, K, n, m);
  if (rc) return rc;
  uint8_t keep[256];
  for (int64_t r0 = 0; r0 < R; r0 += m)
    for (int64_t c0 = 0; c0 < K; c0 += m) {
      greedy_block(W, dt, K, r0, c0, n, m, keep);
      for (int e = 0; e < m * m; e++) {
        int64_t i = (r0 + e / m) * K + c0 + e % m;
        if (keep[e])
          copy_elem(W_out, W, dt, i);
        else
          zero_elem(W_out, dt, i);
      }
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Channel permutation ([ASDNN] "Step-2: Weight Pruning", Fig. 6): permuting  */
/* the columns of W before the N:M mask is taken changes which weights share */
/* a group, and a good permutation keeps a larger total magnitude.  The      */
/* pages show the effect only; the search here is a reading (see            */
/* nm_oracle.h): rounds of pairwise column swaps between groups.             */
/*                                                                           */
/* perm[i] is the column of W placed at position i; groups are positions    */
/* g*m .. g*m+m-1.  All sums are in double over ascending rows.              */
/* ------------------------------------------------------------------------ */

/* sum of the n largest of v[0..m-1] (plain selection sort of a copy) */
static double top_n_sum(const double* v, int n, int m) {
  double c[16];
  for (int i = 0; i < m; i++) c[i] = v[i];
  double s = 0.0;
  for (int k = 0; k < n; k++) {
    int best = k;
    for (int i = k + 1; i < m; i++)
      if (c[i] > c[best]) best = i;
    double t = c[k];
    c[k] = c[best];
    c[best] = t;
    s += c[k];
  }
  return s;
}

static double mag_at(const void* W, int dt, int64_t K, int64_t r, int64_t col) {
  double x = fabs(nmo_to_double(W, dt, r * K + col));
  return isnan(x) ? INFINITY : x;
}

static int check_perm(const int32_t* perm, int64_t K) {
  for (int64_t i = 0; i < K; i++)
    if (perm[i] < 0 || perm[i] >= K) return -6;
  return 0;
}

double nmo_kept_l1(const void* W, int dt, int64_t R, int64_t K, int n, int m,
                   const int32_t* perm) {
  if (check_args(dt, R, K, n, m) || check_perm(perm, K)) return -1.0;
  double total = 0.0, v[16];
  for (int64_t r = 0; r < R; r++)
    for (int64_t g = 0; g < K / m; g++) {
      for (int i = 0; i < m; i++) v[i] = mag_at(W, dt, K, r, perm[g * m + i]);
      total += top_n_sum(v, n, m);
    }
  return total;
}

/* For every pair of groups g1 < g2: the change of the kept L1 caused by swapping the     */
/* column at position a of g1 with the column at position b of g2, summed over all rows,  */
/* maximised over (a, b) (the first (a, b) in row-major order on ties).  gain[g1*G + g2]  */
/* and pick[g1*G + g2] = a*m + b; entries with g1 >= g2 are left as they are.            */
int nmo_perm_gains(const void* W, int dt, int64_t R, int64_t K, int n, int m,
                   const int32_t* perm, double* gain, int32_t* pick) {
  int rc = check_args(dt, R, K, n, m);
  if (rc) return rc;
  if ((rc = check_perm(perm, K))) return rc;
  const int64_t G = K / m;
  double* delta = (double*)malloc(sizeof(double) * (size_t)(m * m));
  if (!delta) return -5;
  double u[16], v[16], u2[16], v2[16];
  for (int64_t g1 = 0; g1 < G; g1++)
    for (int64_t g2 = g1 + 1; g2 < G; g2++) {
      for (int s = 0; s < m * m; s++) delta[s] = 0.0;
      for (int64_t r = 0; r < R; r++) {
        for (int i = 0; i < m; i++) {
          u[i] = mag_at(W, dt, K, r, perm[g1 * m + i]);
          v[i] = mag_at(W, dt, K, r, perm[g2 * m + i]);
        }
        const double base = top_n_sum(u, n, m) + top_n_sum(v, n, m);
        for (int a = 0; a < m; a++)
          for (int b = 0; b < m; b++) {
            for (int i = 0; i < m; i++) {
              u2[i] = u[i];
              v2[i] = v[i];
            }
            u2[a] = v[b];
            v2[b] = u[a];
            delta[a * m + b] += top_n_sum(u2, n, m) + top_n_sum(v2, n, m) - base;
          }
      }
      int best = 0;
      for (int s = 1; s < m * m; s++)
        if (delta[s] > delta[best]) best = s;
      gain[g1 * G + g2] = delta[best];
      pick[g1 * G + g2] = best;
    }
  free(delta);
  return 0;
}

/* Rounds of swaps: compute every pair's best gain; take the pairs with a positive gain  */
/* in descending order of gain (ties: smaller g1, then smaller g2) and apply each one    */
/* whose two groups are still untouched in this round; stop when a round applies none   */
/* or after max_rounds.  perm is updated in place; *rounds_done counts applied rounds.   */
int nmo_perm_search(const void* W, int dt, int64_t R, int64_t K, int n, int m, int max_rounds,
                    int32_t* perm, int* rounds_done) {
  int rc = check_args(dt, R, K, n, m);
  if (rc) return rc;
  if ((rc = check_perm(perm, K))) return rc;
  const int64_t G = K / m;
  double* gain = (double*)malloc(sizeof(double) * (size_t)(G * G > 0 ? G * G : 1));
  int32_t* pick = (int32_t*)malloc(sizeof(int32_t) * (size_t)(G * G > 0 ? G * G : 1));
  uint8_t* used = (uint8_t*)malloc((size_t)(G > 0 ? G : 1));
  if (!gain || !pick || !used) {
    free(gain);
    free(pick);
    free(used);
    return -5;
  }
  int done = 0;
  for (int round = 0; round < max_rounds; round++) {
    nmo_perm_gains(W, dt, R, K, n, m, perm, gain, pick);
    for (int64_t g = 0; g < G; g++) used[g] = 0;
    int applied = 0;
    for (;;) { /* pick the best remaining pair among untouched groups */
      int64_t bg1 = -1, bg2 = -1;
      for (int64_t g1 = 0; g1 < G; g1++) {
        if (used[g1]) continue;
        for (int64_t g2 = g1 + 1; g2 < G; g2++) {
          if (used[g2] || !(gain[g1 * G + g2] > 0.0)) continue;
          if (bg1 < 0 || gain[g1 * G + g2] > gain[bg1 * G + bg2]) {
            bg1 = g1;
            bg2 = g2;
          }
        }
      }
      if (bg1 < 0) break;
      const int s = pick[bg1 * G + bg2], a = s / m, b = s % m;
      const int32_t t = perm[bg1 * m + a];
      perm[bg1 * m + a] = perm[bg2 * m + b];
      perm[bg2 * m + b] = t;
      used[bg1] = used[bg2] = 1;
      applied++;
    }
    if (!applied) break;
    done++;
  }
  free(gain);
  free(pick);
  free(used);
  if (rounds_done) *rounds_done = done;
  return 0;
}
