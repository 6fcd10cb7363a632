/*
 * mk_oracle.c -- TEST INFRASTRUCTURE ONLY. Plain, slow CPU reference for the
 * GEMM+AllReduce kernel of "mKernel: Fast Multi-GPU, Multi-Node Fused Kernels"
 * (arXiv 2609.13585), restricted to one GPU's share of the work.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. The product (libmk.so and its Python binding) never does.
 *
 * What it computes (thelatestinai.com page, Table 3, row "GEMM + AllReduce (TP)":
 * the kernel is compute -> communication and the intra-node step is a reduction
 * of the output tiles across GPUs; tensor parallelism splits K, so every GPU
 * holds a partial product of the full output). For one GPU's share:
 *
 *     C_exact[i,j] = sum_{k < K} A[i,k] * B[k,j]  +  sum_{p < P-1} peer_p[i,j]
 *
 * with A[M,K] and B[K,N] bfloat16 row-major, peers a contiguous [P-1, M, N]
 * array of bfloat16 or float32, and C[M,N] rounded to bfloat16 or float32.
 * The pages give neither the dtypes nor the layout; the readings taken are:
 *   - reduction = plain sum, no scaling;
 *   - dense row-major, peers contiguous;
 *   - output rounding = round to nearest, ties to even.
 *
 * Arithmetic, in this order, per output element:
 *   1. S = sum of the peer values, computed exactly (error-free expansion,
 *      Shewchuk 1997, "Adaptive Precision Floating-Point Arithmetic and Fast
 *      Robust Geometric Predicates") and rounded once to double. S therefore
 *      does not depend on peer order.
 *   2. G = sum over ascending k of A[i,k]*B[k,j] in double. Every bf16*bf16
 *      product is exact in double (8+8 significant bits), so only the additions
 *      round.
 *   3. C64 = G + S (one double rounding).
 *   4. C_out = RNE(C64) to the output type. For bfloat16 this file carries its
 *      own bit-level rounding; for float32 the C conversion (round to nearest
 *      even in the default rounding mode) is used.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { MKO_BF16 = 0, MKO_F32 = 1 };

/* Planted-mistake builds for the test suite's sensitivity check: building with
 * -DMKO_MUTANT=n injects one deliberate error, and the pins must reject every
 * such build. The committed library is built with MKO_MUTANT == 0. */
#ifndef MKO_MUTANT
#define MKO_MUTANT 0
#endif
#define MUT(n) (MKO_MUTANT == (n))

/* bfloat16 bits -> double. A bfloat16 is the upper half of an IEEE binary32, so
 * widening is exact: place the 16 bits in the high half of a float. */
double mko_bf16_to_f64(uint16_t h) {
  uint32_t u = ((uint32_t)(MUT(8) ? (h & 0xFFFEu) : h)) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double f32_bits_to_f64(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* double -> bfloat16 bits, round to nearest, ties to even, straight from the
 * double (a single rounding; no detour through float, which would round twice).
 * bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
 * NaN maps to a quiet NaN with the sign kept; overflow rounds to infinity. */
uint16_t mko_f64_to_bf16_rne(double x) {
  uint64_t u;
  memcpy(&u, &x, 8);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  int e = (int)((u >> 52) & 0x7FF);
  uint64_t frac = u & ((1ull << 52) - 1);
  if (e == 0x7FF) return (uint16_t)(sign | (frac ? 0x7FC0u : 0x7F80u));
  if (e == 0 && frac == 0) return sign;
  /* |x| = sig * 2^(exp2) with sig an integer of 53 bits (normal) or fewer. */
  uint64_t sig;
  int exp2;
  if (e == 0) { sig = frac; exp2 = -1074; }
  else { sig = frac | (1ull << 52); exp2 = e - 1075; }
  /* Position of the leading bit: value = 1.f * 2^lead. */
  int msb = 63 - __builtin_clzll(sig);
  int lead = exp2 + msb;
  /* Target quantum: normal bf16 keeps 8 significant bits -> quantum 2^(lead-7);
   * below 2^-126 the quantum is fixed at 2^-133 (subnormals). */
  int q = lead - 7;
  if (q < -133) q = -133;
  int shift = q - exp2; /* number of low bits of sig to drop */
  uint64_t m;           /* result = m * 2^q */
  if (shift <= 0) {
    m = sig << (-shift); /* exact (only happens for tiny shift counts) */
  } else if (shift >= 64) {
    m = 0; /* far below half a quantum */
  } else {
    uint64_t kept = sig >> shift;
    uint64_t rem = sig & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && ((kept & 1ull) || MUT(5)))) kept += 1;
    m = kept;
  }
  if (m == 0) return sign;
  /* Normalise m * 2^q into bf16 fields. m has at most 9 bits (after a carry). */
  int mmsb = 63 - __builtin_clzll(m);
  int vlead = q + mmsb; /* exponent of the leading bit of the rounded value */
  if (vlead > 127) return (uint16_t)(sign | 0x7F80u); /* overflow -> inf */
  if (vlead < -126) {
    /* subnormal: value = m * 2^-133, fraction field = m (m < 128) */
    return (uint16_t)(sign | (uint16_t)m);
  }
  /* normal: m has exactly 8 significant bits aligned so that leading is 2^vlead */
  uint64_t mant;
  if (mmsb >= 7) mant = m >> (mmsb - 7);
  else mant = m << (7 - mmsb);
  uint16_t ebits = (uint16_t)(vlead + 127);
  return (uint16_t)(sign | (ebits << 7) | (uint16_t)(mant & 0x7Fu));
}

/* Exact sum of n doubles (n <= 64), rounded once to nearest-even. Keeps a list
 * of non-overlapping partials whose exact sum equals the running total (each
 * addition is split into its rounded sum and the exact rounding error by the
 * two-sum transformation; Shewchuk 1997, above), then adds the partials from the
 * largest down and corrects the single case where that last rounding lands on a
 * tie. The partial list with the final half-way correction is the form of
 * Raymond Hettinger's "msum" recipe (ActiveState Python Cookbook, recipe
 * 393090), which CPython's math.fsum also follows. Each input adds at most one
 * partial, so n <= 64 values never need more than 64 partials. */
#define MKO_MAX_PARTIALS 64 /* non-overlapping partials of doubles: about 40 at most */
#define MKO_MAX_PEERS 64    /* peer values held per output element */
static double exact_sum(const double* x, int n) {
  double p[MKO_MAX_PARTIALS];
  int np = 0;
  for (int a = 0; a < n; a++) {
    double v = x[a];
    int w = 0;
    for (int b = 0; b < np; b++) {
      double y = p[b];
      if (fabs(v) < fabs(y)) { double t = v; v = y; y = t; }
      double hi = v + y;
      double lo = y - (hi - v); /* exact because |v| >= |y| */
      if (lo != 0.0) p[w++] = lo;
      v = hi;
    }
    p[w++] = v; /* np never exceeds the number of binades spanned (< 64) */
    np = w;
  }
  if (np == 0) return 0.0;
  /* p[] holds increasing magnitudes, non-overlapping. Sum from the top. */
  int i = np - 1;
  double hi = p[i];
  double lo = 0.0;
  while (i > 0) {
    double v = hi;
    double y = p[--i];
    hi = v + y;
    double yr = hi - v;
    lo = y - yr;
    if (lo != 0.0) break;
  }
  /* If the rest is a tie-breaker, nudge towards it. */
  if (!MUT(9) && i > 0 && ((lo < 0.0 && p[i - 1] < 0.0) || (lo > 0.0 && p[i - 1] > 0.0))) {
    double y = lo * 2.0;
    double v = hi + y;
    double yr = v - hi;
    if (y == yr) hi = v;
  }
  return hi;
}

double mko_exact_sum(const double* x, int n) { return exact_sum(x, n); }

static double peer_value(const void* peers, int dtype, int64_t idx) {
  if (dtype == MKO_BF16) return mko_bf16_to_f64(((const uint16_t*)peers)[idx]);
  return f32_bits_to_f64(((const uint32_t*)peers)[idx]);
}

/*
 * mko_gemm_ar: the reference for selected rows.
 *   A      : [M,K] bfloat16 bits, row-major
 *   B      : [K,N] bfloat16 bits, row-major
 *   peers  : [n_peers, M, N] of peer_dtype (may be NULL when n_peers == 0)
 *   rows   : n_rows row indices into [0,M); NULL means all rows (n_rows = M)
 *   C64    : [n_rows, N] double output (may be NULL)
 *   C_out  : [n_rows, N] output of c_dtype (may be NULL)
 *   n_threads : OpenMP threads, <= 0 means the runtime default
 * Returns 0 on success, -1 on bad arguments.
 */
int mko_gemm_ar(const uint16_t* A, const uint16_t* B, const void* peers, int n_peers,
                int peer_dtype, int64_t M, int64_t N, int64_t K, const int64_t* rows,
                int64_t n_rows, double* C64, void* C_out, int c_dtype, int n_threads) {
  if (M < 0 || N < 0 || K < 0 || n_peers < 0 || n_peers > MKO_MAX_PEERS) return -1;
  if ((K > 0 && (!A || !B)) || (n_peers > 0 && !peers)) return -1;
  if (peer_dtype != MKO_BF16 && peer_dtype != MKO_F32) return -1;
  if (c_dtype != MKO_BF16 && c_dtype != MKO_F32) return -1;
  if (!rows) n_rows = M;
  for (int64_t r = 0; r < (rows ? n_rows : 0); r++)
    if (rows[r] < 0 || rows[r] >= M) return -1;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
  int status = 0;
#pragma omp parallel
  {
    double* G = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double pv[MKO_MAX_PEERS];
    if (!G) {
#pragma omp atomic write
      status = -1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < n_rows; r++) {
        int64_t i = rows ? (MUT(7) ? (rows[r] + 1) % M : rows[r]) : r;
        /* step 2: G = sum over ascending k of A[i,k] * B[k,:] */
        for (int64_t j = 0; j < N; j++) G[j] = 0.0;
        for (int64_t k = 0; k < (MUT(4) ? K - 1 : K); k++) {
          double a = mko_bf16_to_f64(A[i * K + k]);
          const uint16_t* brow = B + k * N;
          for (int64_t j = 0; j < N; j++) G[j] += a * mko_bf16_to_f64(brow[MUT(2) ? N - 1 - j : j]);
        }
        for (int64_t j = 0; j < N; j++) {
          /* step 1: exact peer sum S */
          int np_used = MUT(1) && n_peers > 0 ? n_peers - 1 : n_peers;
          for (int p = 0; p < np_used; p++)
            pv[p] = peer_value(peers, peer_dtype, ((int64_t)p * M + i) * N + j);
          double S = exact_sum(pv, np_used);
          /* step 3 */
          double c = MUT(3) ? G[j] - S : G[j] + S;
          if (MUT(6)) { c = G[j]; for (int p = 0; p < np_used; p++) c += pv[p]; }
          if (C64) C64[r * N + j] = c;
          /* step 4 */
          if (C_out) {
            if (c_dtype == MKO_BF16) ((uint16_t*)C_out)[r * N + j] = mko_f64_to_bf16_rne(c);
            else ((float*)C_out)[r * N + j] = MUT(10) ? (float)G[j] + (float)S : (float)c;
          }
        }
      }
      free(G);
    }
  }
  return status;
}

/* Threads OpenMP would use, for reporting. */
int mko_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Array helpers for the test harness. */
void mko_bf16_to_f64_array(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = mko_bf16_to_f64(in[i]);
}
void mko_f64_to_bf16_array(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = mko_f64_to_bf16_rne(in[i]);
}
