/*
 * Plain C oracle for the exact long-accumulator GEMM.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * cpu_baseline leg of the benchmark, never by the product library.  It shares
 * no code with the HIP path.
 *
 * What it computes follows the det-train page, "Method" section: each product
 * x[m,k]*w[n,k] is exact (bf16 and f32 significands multiply exactly), its
 * base-2^32 limbs are added with the product's sign into a per-output array of
 * signed int64 digits, and the exact sum is rounded once to fp32.  Shapes and
 * limits follow the "Usage" and "Requirements and limits" sections: x is
 * [M, K], w is [N, K], K <= 2^19, inputs are bf16 or f32.
 *
 * Layout reading (the page gives none): 18 digits per output, digit j weighs
 * 2^(32*j - 298); digits are raw sums (no carries before rounding).  Rounding
 * is IEEE binary32 round-to-nearest-even with gradual underflow and overflow
 * to +-inf; an exact zero gives +0.0, a nonzero sum keeps its sign.
 *
 * Deliberately plain: one output at a time, one product at a time, 128-bit
 * shifts, no blocking.  Threads split the list of outputs.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ND 18           /* digits per output */
#define LSB 298         /* digit 0 weighs 2^-298 */
#define KMAX (1L << 19)

enum { OR_OK = 0, OR_EKLIMIT = -1, OR_ENONFINITE = -2, OR_ERANGE = -3,
       OR_EOVERFLOW = -4, OR_EINVAL = -5, OR_ENOMEM = -6 };

typedef struct { uint32_t m; int32_t ex; int32_t neg; } dec_t;

/* value = (-1)^neg * m * 2^ex; subnormals keep their fraction (no flush). */
static int decode(int dtype, const void* base, long idx, dec_t* d) {
  if (dtype == 0) {
    uint32_t b = ((const uint32_t*)base)[idx];
    uint32_t e = (b >> 23) & 0xFFu, f = b & 0x7FFFFFu;
    if (e == 0xFFu) return OR_ENONFINITE;
    d->neg = (int32_t)(b >> 31);
    if (e == 0) { d->m = f; d->ex = -149; }
    else { d->m = f | (1u << 23); d->ex = (int32_t)e - 150; }
  } else {
    uint16_t b = ((const uint16_t*)base)[idx];
    uint32_t e = (b >> 7) & 0xFFu, f = b & 0x7Fu;
    if (e == 0xFFu) return OR_ENONFINITE;
    d->neg = (int32_t)(b >> 15);
    if (e == 0) { d->m = f; d->ex = -133; }
    else { d->m = f | (1u << 7); d->ex = (int32_t)e - 134; }
  }
  return OR_OK;
}

static int decode_row(int dtype, const void* base, long ld, long row, long K, dec_t* out) {
  for (long k = 0; k < K; ++k) {
    int rc = decode(dtype, base, row * ld + k, &out[k]);
    if (rc) return rc;
  }
  return OR_OK;
}

/* Raw digits of one output: limb i of |product| goes, signed, into digit d+i. */
static int partial_one(const dec_t* xr, const dec_t* wr, long K, int64_t* dig) {
  memset(dig, 0, ND * sizeof(int64_t));
  for (long k = 0; k < K; ++k) {
    uint64_t M = (uint64_t)xr[k].m * (uint64_t)wr[k].m;
    if (M == 0) continue;
    int o = xr[k].ex + wr[k].ex + LSB;
    int d = o >> 5, s = o & 31;
    unsigned __int128 T = (unsigned __int128)M << s;
    int neg = xr[k].neg ^ wr[k].neg;
    for (int i = 0; T != 0; ++i, T >>= 32) {
      int64_t limb = (int64_t)(uint64_t)(T & 0xFFFFFFFFu);
      if (limb == 0) continue;
      if (d + i >= ND) return OR_ERANGE;
      dig[d + i] += neg ? -limb : limb;
    }
  }
  return OR_OK;
}

/* ---- rounding of the digit value to binary32 ---- */

/* bits [lo, lo+len) of a little-endian array of 32-bit words, len <= 32 */
static uint32_t get_bits(const uint32_t* w, int nw, int lo, int len) {
  uint64_t acc = 0;
  int wi = lo >> 5, sh = lo & 31;
  if (wi < nw) acc = w[wi];
  if (wi + 1 < nw) acc |= (uint64_t)w[wi + 1] << 32;
  acc >>= sh;
  return (uint32_t)(acc & (len == 32 ? 0xFFFFFFFFull : ((1ull << len) - 1)));
}

static int any_bits_below(const uint32_t* w, int nw, int pos) { /* bits [0,pos) */
  int full = pos >> 5;
  for (int i = 0; i < full && i < nw; ++i) if (w[i]) return 1;
  int rem = pos & 31;
  if (rem && full < nw && (w[full] & ((1u << rem) - 1))) return 1;
  return 0;
}

uint32_t oracle_finalize_one(const int64_t* dig) {
  /* carry-propagate the signed digits into 32-bit words plus a signed top */
  uint32_t w[ND + 1];
  __int128 carry = 0;
  for (int j = 0; j < ND; ++j) {
    __int128 t = (__int128)dig[j] + carry;
    w[j] = (uint32_t)(t & 0xFFFFFFFF);
    carry = t >> 32;   /* floor division by 2^32 */
  }
  int negative = carry < 0;
  if (negative) {      /* redo with negated digits to get the magnitude */
    carry = 0;
    for (int j = 0; j < ND; ++j) {
      __int128 t = -(__int128)dig[j] + carry;
      w[j] = (uint32_t)(t & 0xFFFFFFFF);
      carry = t >> 32;
    }
  }
  w[ND] = (uint32_t)carry;   /* magnitude < 2^608 for any digits in range */
  int nw = ND + 1, top = -1;
  for (int j = nw - 1; j >= 0; --j) if (w[j]) { top = j; break; }
  if (top < 0) return 0u;    /* exact zero: +0.0 */
  int n = 32 * top + (32 - __builtin_clz(w[top]));   /* bit length of |I| */
  int q = n - 24 > 149 ? n - 24 : 149;               /* lowest kept bit */
  uint32_t r = get_bits(w, nw, q, n - q > 0 ? n - q : 0);
  if (n - q <= 0) r = 0;
  int half = get_bits(w, nw, q - 1, 1) != 0;
  int sticky = any_bits_below(w, nw, q - 1);
  if (half && (sticky || (r & 1u))) r += 1;
  if (r == (1u << 24)) { r = 1u << 23; q += 1; }
  uint32_t mag;
  if (r < (1u << 23)) mag = r;                       /* subnormal or zero */
  else {
    int E = q - 148;
    mag = E >= 255 ? 0x7F800000u : ((uint32_t)E << 23) | (r - (1u << 23));
  }
  return ((uint32_t)negative << 31) | mag;
}

void oracle_finalize(const int64_t* dig, long n, uint32_t* out) {
  for (long i = 0; i < n; ++i) out[i] = oracle_finalize_one(dig + i * ND);
}

int oracle_combine(const int64_t* const* parts, int nparts, long nvals, int64_t* out) {
  if (nparts < 1) return OR_EINVAL;
  for (long i = 0; i < nvals; ++i) {
    int64_t acc = 0;
    for (int p = 0; p < nparts; ++p)
      if (__builtin_add_overflow(acc, parts[p][i], &acc)) return OR_EOVERFLOW;
    out[i] = acc;
  }
  return OR_OK;
}

/* ---- threaded drivers ---- */

typedef struct {
  int dtype; const void* x; long ldx; const void* w; long ldw; long K;
  const long* rows; const long* cols; long npairs;   /* pair mode */
  long M, N;                                          /* full mode when rows == NULL */
  int64_t* out; int tid, nthreads; int rc;
} job_t;

static void* run_job(void* arg) {
  job_t* j = (job_t*)arg;
  j->rc = OR_OK;
  dec_t* xr = (dec_t*)malloc(sizeof(dec_t) * (size_t)(j->K > 0 ? j->K : 1));
  dec_t* wr = (dec_t*)malloc(sizeof(dec_t) * (size_t)(j->K > 0 ? j->K : 1));
  if (!xr || !wr) { free(xr); free(wr); j->rc = OR_ENOMEM; return NULL; }
  if (j->rows) {
    for (long p = j->tid; p < j->npairs && !j->rc; p += j->nthreads) {
      int rc = decode_row(j->dtype, j->x, j->ldx, j->rows[p], j->K, xr);
      if (!rc) rc = decode_row(j->dtype, j->w, j->ldw, j->cols[p], j->K, wr);
      if (!rc) rc = partial_one(xr, wr, j->K, j->out + p * ND);
      j->rc = rc;
    }
  } else {
    for (long m = j->tid; m < j->M && !j->rc; m += j->nthreads) {
      int rc = decode_row(j->dtype, j->x, j->ldx, m, j->K, xr);
      for (long n = 0; n < j->N && !rc; ++n) {
        rc = decode_row(j->dtype, j->w, j->ldw, n, j->K, wr);
        if (!rc) rc = partial_one(xr, wr, j->K, j->out + (m * j->N + n) * ND);
      }
      j->rc = rc;
    }
  }
  free(xr); free(wr);
  return NULL;
}

static int run_threads(job_t proto, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) { free(jobs); free(th); return OR_ENOMEM; }
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = proto; jobs[t].tid = t; jobs[t].nthreads = nthreads;
    pthread_create(&th[t], NULL, run_job, &jobs[t]);
  }
  int rc = OR_OK;
  for (int t = 0; t < nthreads; ++t) {
    pthread_join(th[t], NULL);
    if (jobs[t].rc && !rc) rc = jobs[t].rc;
  }
  free(jobs); free(th);
  return rc;
}

/* Raw digits of the whole [M, N] output: out is [M][N][18]. */
int oracle_partial_full(int dtype, const void* x, long ldx, const void* w, long ldw,
                        long M, long N, long K, int64_t* out, int nthreads) {
  if (K > KMAX) return OR_EKLIMIT;
  if (M < 0 || N < 0 || K < 0 || (dtype != 0 && dtype != 1)) return OR_EINVAL;
  job_t j; memset(&j, 0, sizeof j);
  j.dtype = dtype; j.x = x; j.ldx = ldx; j.w = w; j.ldw = ldw; j.K = K;
  j.M = M; j.N = N; j.out = out;
  return run_threads(j, nthreads);
}

/* Raw digits of selected outputs (rows[p], cols[p]): out is [npairs][18]. */
int oracle_partial_pairs(int dtype, const void* x, long ldx, const void* w, long ldw,
                         long K, const long* rows, const long* cols, long npairs,
                         int64_t* out, int nthreads) {
  if (K > KMAX) return OR_EKLIMIT;
  if (npairs < 0 || K < 0 || (dtype != 0 && dtype != 1)) return OR_EINVAL;
  if (npairs == 0) return OR_OK;
  job_t j; memset(&j, 0, sizeof j);
  j.dtype = dtype; j.x = x; j.ldx = ldx; j.w = w; j.ldw = ldw; j.K = K;
  j.rows = rows; j.cols = cols; j.npairs = npairs; j.out = out;
  return run_threads(j, nthreads);
}
