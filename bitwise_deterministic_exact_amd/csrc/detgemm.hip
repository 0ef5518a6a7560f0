// Exact long-accumulator GEMM for MI355X (gfx950): kernels and the C ABI.
//
// Follows the det-train page: "Method" (exact products, base-2^32 limbs added
// into signed int64 digits of a Kulisch accumulator, one rounding to fp32),
// "Usage" (det_gemm / det_gemm_partial / det_combine / det_finalize on x[M,K]
// and w[N,K] and their K-slices) and "Requirements and limits" (K <= 2^19,
// bf16 and f32).  The accumulator layout and rounding are documented in
// include/detgemm.h.
//
// The accumulate step is exact integer work, so it runs on the vector ALUs and
// the LDS, not on the matrix cores:
//   * a workgroup of 256 lanes owns a 16x16 tile of outputs, one per lane;
//   * operands are staged per K-chunk into LDS already decoded into an integer
//     significand and a packed exponent/sign word;
//   * every lane keeps its output's digits in LDS as two raw sums per digit
//     (products of either sign), laid out [slot][lane] so that the 64 lanes of
//     a wave hit distinct banks; each product's limbs go in with ds_add_u64,
//     whose address is the only per-lane dynamic index the hardware offers;
//   * the epilogue subtracts the two sums and either writes the raw digits or
//     rounds them in registers to fp32.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "detgemm.h"

namespace {

constexpr int ND = DET_NUM_DIGITS;   // 18 digits per output
constexpr int TILE = 16;             // outputs per tile edge
constexpr int NT = TILE * TILE;      // lanes per workgroup, one output each
constexpr int KC = 16;               // K values staged per chunk
constexpr int NSLOT = 2 * ND;        // digit sums of positive and of negative products
constexpr int COMBINE_MAX = 32;      // parts summed per combine launch

thread_local char g_err[512];

det_status fail(det_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

det_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DET_EHIP, "%s: %s", what, hipGetErrorString(e));
  return DET_OK;
}

// ---------------------------------------------------------------- decode
//
// An operand element becomes {m, e}: m is the integer significand (hidden bit
// included for normal numbers, raw fraction for subnormals, never flushed) and
// e packs an exponent offset in bits 0..9 and the sign in bit 11.  The
// offsets are chosen so that for a product of two elements, with
// sum = e_x + e_w,
//     o = sum & 1023 = ex + ew + 298
// is the bit position of the product's least significant bit in the digit
// array (value = m_x*m_w * 2^(o - 298)), and bit 11 of sum is the product's
// sign (offsets stay below 1024, so nothing carries into bit 11).
//   f32 : value = m * 2^(max(E,1) - 150)  ->  offset = max(E,1) - 1
//   bf16: value = m * 2^(max(E,1) - 134)  ->  offset = max(E,1) + 15
// For every bit pattern (Inf and NaN included) o <= 540, so the limbs of any
// product land in digits 0..17: no input can index outside the array.
constexpr uint32_t SIGN_BIT = 11;

template <int DT>
__device__ __forceinline__ uint2 decode_elem(const void* __restrict__ base, int64_t idx, bool valid) {
  if (!valid) return make_uint2(0u, 0u);
  if (DT == DET_F32) {
    const uint32_t b = static_cast<const uint32_t*>(base)[idx];
    const uint32_t E = (b >> 23) & 0xFFu;
    const uint32_t m = (b & 0x7FFFFFu) | (min(E, 1u) << 23);
    const uint32_t e = (max(E, 1u) - 1u) | ((b >> 31) << SIGN_BIT);
    return make_uint2(m, e);
  } else {
    const uint32_t b = static_cast<const uint16_t*>(base)[idx];
    const uint32_t E = (b >> 7) & 0xFFu;
    const uint32_t m = (b & 0x7Fu) | (min(E, 1u) << 7);
    const uint32_t e = (max(E, 1u) + 15u) | ((b >> 15) << SIGN_BIT);
    return make_uint2(m, e);
  }
}

// ---------------------------------------------------------------- rounding
//
// Round the value sum_j dg[j] * 2^(32 j - 298) once to binary32 (nearest,
// ties to even, gradual underflow, overflow to inf; exact zero -> +0).
// Precondition |dg[j]| <= 2^62.  Fully unrolled: every index is static, so the
// 18 words stay in registers.
__device__ uint32_t round_digits_to_f32(const int64_t (&dg)[ND]) {
  uint32_t w[ND];
  int64_t carry = 0;
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    const int64_t t = dg[j] + carry;
    w[j] = static_cast<uint32_t>(t);
    carry = t >> 32;                  // arithmetic: floor(t / 2^32)
  }
  // value = W + carry * 2^576 with W = sum w[j] 2^(32j)
  if (carry != 0 && carry != -1) return carry < 0 ? 0xFF800000u : 0x7F800000u;
  const bool neg = carry < 0;
  if (neg) {                          // |value| = 2^576 - W
    uint32_t c = 1u;
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const uint32_t v = ~w[j] + c;
      c = (c != 0u && v == 0u) ? 1u : 0u;
      w[j] = v;
    }
    if (c) return 0xFF800000u;        // |value| = 2^576
  }
  int top = -1;
  uint32_t wt = 0u;
#pragma unroll
  for (int j = 0; j < ND; ++j)
    if (w[j] != 0u) { top = j; wt = w[j]; }
  if (top < 0) return 0u;             // exact zero: +0.0
  const int n = 32 * top + 32 - __clz(static_cast<int>(wt));   // bit length of |value|
  int q = max(n - 24, 149);           // lowest kept bit (2^-149 = bit 149)
  const int a = (q - 1) >> 5, sh = (q - 1) & 31;
  uint32_t wa = 0u, wb = 0u;
  bool below = false;
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    if (j == a) wa = w[j];
    if (j == a + 1) wb = w[j];
    if (j < a && w[j] != 0u) below = true;
  }
  const uint64_t win = (static_cast<uint64_t>(wb) << 32) | wa;
  const uint64_t v = win >> sh;                       // bit 0: half bit, above: r
  const bool sticky = below || (win & ((1ull << sh) - 1ull)) != 0ull;
  uint32_t r = static_cast<uint32_t>(v >> 1) & 0x1FFFFFFu;
  if ((v & 1ull) && (sticky || (r & 1u))) r += 1u;
  if (r == (1u << 24)) { r = 1u << 23; q += 1; }
  uint32_t mag;
  if (r < (1u << 23)) {
    mag = r;                                          // subnormal (q == 149) or zero
  } else {
    const int E = q - 148;
    mag = E >= 255 ? 0x7F800000u : (static_cast<uint32_t>(E) << 23) | (r - (1u << 23));
  }
  return (neg ? 0x80000000u : 0u) | mag;
}

// ---------------------------------------------------------------- GEMM kernel
struct GemmArgs {
  const void* x; int64_t x_sm, x_sk;
  const void* w; int64_t w_sn, w_sk;
  int64_t M, N, K;
  int64_t tiles_n;
  int64_t* acc;                       // partial: [M][N][18]
  float* y; int64_t y_sm, y_sn;       // gemm: fp32 out
};

// Per-lane digit sums in LDS, byte address
//     lane*8 + sign*2048 + digit*4096
// i.e. [digit][sign][lane] with 256 lanes of 8 bytes.  Digit and sign move an
// address by multiples of 2048 bytes, so the bank a lane hits depends only on
// the lane: a wave's atomics spread over all banks whatever its digits are.
constexpr int SIGN_STRIDE = NT * 8;          // 2048 bytes
constexpr int DIGIT_STRIDE = 2 * NT * 8;     // 4096 bytes
constexpr int KPAD = KC + 2;                 // staging row pitch (uint2), keeps b128 reads conflict-free

// Add one exact product into the lane's digit sums.
template <int DT>
__device__ __forceinline__ void accumulate(char* lds_lane, uint2 xv, uint2 wv) {
  const uint32_t sum = xv.y + wv.y;
  const uint32_t s = sum & 31u;                                  // shift inside the digit
  const uint32_t d = (sum >> 5) & 31u;                           // first digit
  const uint32_t off = (d << 12) | (sum & (1u << SIGN_BIT));     // digit*4096 + sign*2048
  unsigned long long* p = reinterpret_cast<unsigned long long*>(lds_lane + off);
  const uint64_t M = static_cast<uint64_t>(xv.x) * wv.x;         // exact significand product
  const uint64_t lo = M << s;                                    // limbs 0 and 1
  atomicAdd(p, static_cast<unsigned long long>(static_cast<uint32_t>(lo)));
  atomicAdd(p + DIGIT_STRIDE / 8, static_cast<unsigned long long>(lo >> 32));
  if (DT == DET_F32) {                                           // f32 products reach limb 2
    const uint64_t l2 = (static_cast<uint64_t>(static_cast<uint32_t>(M >> 32)) << s) >> 32;
    atomicAdd(p + 2 * DIGIT_STRIDE / 8, static_cast<unsigned long long>(l2));
  }
}

// OUT = 0: write raw digits; OUT = 1: round to fp32.
template <int DT, int OUT>
__global__ __launch_bounds__(NT) void k_gemm(GemmArgs a) {
  __shared__ __align__(16) unsigned long long sums[NSLOT * NT];   // see the layout above
  __shared__ __align__(16) uint2 xs[TILE][KPAD];     // decoded x chunk [row][k]
  __shared__ __align__(16) uint2 ws[TILE][KPAD];     // decoded w chunk [col][k]

  const int tid = threadIdx.x;
  const int ty = tid / TILE, tx = tid % TILE;
  const int64_t tm = blockIdx.x / a.tiles_n, tn = blockIdx.x % a.tiles_n;
  const int64_t m0 = tm * TILE, n0 = tn * TILE;

#pragma unroll
  for (int s = 0; s < NSLOT; ++s) sums[s * NT + tid] = 0ull;
  char* const lds_lane = reinterpret_cast<char*>(sums) + tid * 8;

  // staging role of this lane: element (row sr, k sc) of the chunk
  const int sr = tid / KC, sc = tid % KC;
  const bool xrow_ok = m0 + sr < a.M, wrow_ok = n0 + sr < a.N;
  const int64_t xrow = xrow_ok ? (m0 + sr) * a.x_sm : 0;
  const int64_t wrow = wrow_ok ? (n0 + sr) * a.w_sn : 0;

  for (int64_t k0 = 0; k0 < a.K; k0 += KC) {
    const int64_t k = k0 + sc;
    const bool kok = k < a.K;
    xs[sr][sc] = decode_elem<DT>(a.x, xrow + k * a.x_sk, xrow_ok && kok);
    ws[sr][sc] = decode_elem<DT>(a.w, wrow + k * a.w_sk, wrow_ok && kok);
    __syncthreads();
    uint4 xq[KC / 2], wq[KC / 2];                    // the whole chunk in registers
#pragma unroll
    for (int i = 0; i < KC / 2; ++i) {
      xq[i] = *reinterpret_cast<const uint4*>(&xs[ty][2 * i]);
      wq[i] = *reinterpret_cast<const uint4*>(&ws[tx][2 * i]);
    }
    __syncthreads();                                 // staging buffer free again
#pragma unroll
    for (int i = 0; i < KC / 2; ++i) {
      accumulate<DT>(lds_lane, make_uint2(xq[i].x, xq[i].y), make_uint2(wq[i].x, wq[i].y));
      accumulate<DT>(lds_lane, make_uint2(xq[i].z, xq[i].w), make_uint2(wq[i].z, wq[i].w));
    }
  }
  __syncthreads();

  const int64_t m = m0 + ty, n = n0 + tx;
  if (m >= a.M || n >= a.N) return;
  const unsigned long long* mine = reinterpret_cast<const unsigned long long*>(lds_lane);
  int64_t dg[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j)
    dg[j] = static_cast<int64_t>(mine[j * (DIGIT_STRIDE / 8)] - mine[j * (DIGIT_STRIDE / 8) + SIGN_STRIDE / 8]);
  if (OUT == 0) {
    int64_t* out = a.acc + (m * a.N + n) * ND;
#pragma unroll
    for (int j = 0; j < ND; ++j) out[j] = dg[j];
  } else {
    const uint32_t bits = round_digits_to_f32(dg);
    a.y[m * a.y_sm + n * a.y_sn] = __uint_as_float(bits);
  }
}

// ---------------------------------------------------------------- combine / finalize
struct CombineArgs {
  const int64_t* parts[COMBINE_MAX];
  int nparts;
  int64_t* out;
  int64_t n;                          // int64 elements
};

__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < a.n; i += stride) {
    int64_t s = 0;
    for (int p = 0; p < a.nparts; ++p) s += a.parts[p][i];
    a.out[i] = s;
  }
}

__global__ __launch_bounds__(256) void k_finalize(const int64_t* __restrict__ acc, float* __restrict__ y,
                                                   int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int64_t dg[ND];
  const int64_t* src = acc + i * ND;
#pragma unroll
  for (int j = 0; j < ND; ++j) dg[j] = src[j];
  y[i] = __uint_as_float(round_digits_to_f32(dg));
}

__global__ __launch_bounds__(256) void k_round_bf16(const uint32_t* __restrict__ in, uint16_t* __restrict__ out,
                                                     int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t b = in[i];
  uint16_t r;
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x7FFFFFu)) {
    r = static_cast<uint16_t>((b >> 16) | 0x40u);            // NaN stays a (quiet) NaN
  } else {
    // nearest-even on the bit pattern: add half an ulp minus one, plus the
    // lowest kept bit, then truncate; exact for every finite value and
    // carries into the exponent (up to Inf) where it must
    r = static_cast<uint16_t>((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
  }
  out[i] = r;
}

template <int DT>
__global__ __launch_bounds__(256) void k_check_finite(const void* __restrict__ p, int64_t rows, int64_t cols,
                                                       int64_t s_row, int64_t s_col, int32_t* flag) {
  const int64_t total = rows * cols;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  bool bad = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t r = i / cols, c = i % cols;
    const int64_t idx = r * s_row + c * s_col;
    if (DT == DET_F32) bad |= (static_cast<const uint32_t*>(p)[idx] & 0x7F800000u) == 0x7F800000u;
    else bad |= (static_cast<const uint16_t*>(p)[idx] & 0x7F80u) == 0x7F80u;
  }
  if (bad) *flag = 1;
}

// ---------------------------------------------------------------- host helpers
det_status check_operands(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk, const void* w,
                          int64_t w_sn, int64_t w_sk, int64_t M, int64_t N, int64_t K) {
  if (dt != DET_F32 && dt != DET_BF16) return fail(DET_EDTYPE, "unknown dtype %d", static_cast<int>(dt));
  if (M < 0 || N < 0 || K < 0) return fail(DET_EINVAL, "negative size M=%lld N=%lld K=%lld",
                                           (long long)M, (long long)N, (long long)K);
  if (K > DET_K_MAX) return fail(DET_EKLIMIT, "K = %lld exceeds the limit 2^19", (long long)K);
  if (x_sm < 0 || x_sk < 0 || w_sn < 0 || w_sk < 0) return fail(DET_EINVAL, "negative stride");
  if (M > 0 && N > 0 && K > 0 && (x == nullptr || w == nullptr)) return fail(DET_EINVAL, "null operand");
  const uintptr_t align = dt == DET_F32 ? 4u : 2u;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w)) & (align - 1))
    return fail(DET_EINVAL, "operands must be aligned to their element size");
  return DET_OK;
}

det_status launch_gemm(det_dtype dt, int out_mode, GemmArgs a, hipStream_t s) {
  const int64_t tiles_m = (a.M + TILE - 1) / TILE;
  a.tiles_n = (a.N + TILE - 1) / TILE;
  const int64_t blocks = tiles_m * a.tiles_n;
  if (blocks == 0) return DET_OK;
  if (blocks > 0x7FFFFFFF) return fail(DET_EINVAL, "too many output tiles");
  const dim3 grid(static_cast<unsigned>(blocks)), block(NT);
  if (dt == DET_F32) {
    if (out_mode == 0) hipLaunchKernelGGL((k_gemm<DET_F32, 0>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm<DET_F32, 1>), grid, block, 0, s, a);
  } else {
    if (out_mode == 0) hipLaunchKernelGGL((k_gemm<DET_BF16, 0>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((k_gemm<DET_BF16, 1>), grid, block, 0, s, a);
  }
  return hip_check(hipGetLastError(), "gemm launch");
}

unsigned grid_for(int64_t n, int64_t per_block, unsigned cap) {
  int64_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return static_cast<unsigned>(g > cap ? cap : g);
}

}  // namespace

// ---------------------------------------------------------------- C ABI
extern "C" {

int det_num_digits(void) { return ND; }
int det_lsb_exponent(void) { return DET_LSB_EXPONENT; }
int64_t det_k_max(void) { return DET_K_MAX; }
const char* det_last_error(void) { return g_err; }

det_status det_gemm(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk, const void* w, int64_t w_sn,
                    int64_t w_sk, int64_t M, int64_t N, int64_t K, float* y, int64_t y_sm, int64_t y_sn,
                    void* stream) {
  det_status st = check_operands(dt, x, x_sm, x_sk, w, w_sn, w_sk, M, N, K);
  if (st != DET_OK) return st;
  if (M > 0 && N > 0 && y == nullptr) return fail(DET_EINVAL, "null output");
  if (y_sm < 0 || y_sn < 0) return fail(DET_EINVAL, "negative output stride");
  if (reinterpret_cast<uintptr_t>(y) & 3u) return fail(DET_EINVAL, "output must be 4-byte aligned");
  GemmArgs a{};
  a.x = x; a.x_sm = x_sm; a.x_sk = x_sk;
  a.w = w; a.w_sn = w_sn; a.w_sk = w_sk;
  a.M = M; a.N = N; a.K = K;
  a.y = y; a.y_sm = y_sm; a.y_sn = y_sn;
  return launch_gemm(dt, 1, a, static_cast<hipStream_t>(stream));
}

det_status det_gemm_partial(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk, const void* w,
                            int64_t w_sn, int64_t w_sk, int64_t M, int64_t N, int64_t K, int64_t* acc,
                            void* stream) {
  det_status st = check_operands(dt, x, x_sm, x_sk, w, w_sn, w_sk, M, N, K);
  if (st != DET_OK) return st;
  if (M > 0 && N > 0 && acc == nullptr) return fail(DET_EINVAL, "null accumulator");
  if (reinterpret_cast<uintptr_t>(acc) & 7u) return fail(DET_EINVAL, "accumulator must be 8-byte aligned");
  GemmArgs a{};
  a.x = x; a.x_sm = x_sm; a.x_sk = x_sk;
  a.w = w; a.w_sn = w_sn; a.w_sk = w_sk;
  a.M = M; a.N = N; a.K = K;
  a.acc = acc;
  return launch_gemm(dt, 0, a, static_cast<hipStream_t>(stream));
}

det_status det_combine(const int64_t* const* parts, int nparts, int64_t* out, int64_t n_outputs,
                       void* stream) {
  if (parts == nullptr || nparts < 1) return fail(DET_EINVAL, "combine needs at least one part");
  if (n_outputs < 0) return fail(DET_EINVAL, "negative output count");
  if (n_outputs == 0) return DET_OK;
  if (out == nullptr) return fail(DET_EINVAL, "null output");
  for (int p = 0; p < nparts; ++p)
    if (parts[p] == nullptr) return fail(DET_EINVAL, "null part %d", p);
  const int64_t n = n_outputs * ND;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // more than COMBINE_MAX parts: fold them in groups, carrying the running sum
  // in `out` (integer addition: any grouping gives the same digits)
  int done = 0;
  while (done < nparts) {
    CombineArgs a{};
    a.out = out;
    a.n = n;
    if (done > 0) a.parts[a.nparts++] = out;
    while (a.nparts < COMBINE_MAX && done < nparts) a.parts[a.nparts++] = parts[done++];
    hipLaunchKernelGGL(k_combine, dim3(grid_for(n, 256, 65536)), dim3(256), 0, s, a);
    det_status st = hip_check(hipGetLastError(), "combine launch");
    if (st != DET_OK) return st;
  }
  return DET_OK;
}

det_status det_finalize(const int64_t* acc, float* y, int64_t n_outputs, void* stream) {
  if (n_outputs < 0) return fail(DET_EINVAL, "negative output count");
  if (n_outputs == 0) return DET_OK;
  if (acc == nullptr || y == nullptr) return fail(DET_EINVAL, "null pointer");
  hipLaunchKernelGGL(k_finalize, dim3(static_cast<unsigned>((n_outputs + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), acc, y, n_outputs);
  return hip_check(hipGetLastError(), "finalize launch");
}

det_status det_round_f32_to_bf16(const float* in, uint16_t* out, int64_t n, void* stream) {
  if (n < 0) return fail(DET_EINVAL, "negative count");
  if (n == 0) return DET_OK;
  if (in == nullptr || out == nullptr) return fail(DET_EINVAL, "null pointer");
  hipLaunchKernelGGL(k_round_bf16, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), reinterpret_cast<const uint32_t*>(in), out, n);
  return hip_check(hipGetLastError(), "round launch");
}

det_status det_check_finite(det_dtype dt, const void* p, int64_t rows, int64_t cols, int64_t s_row,
                            int64_t s_col, int32_t* flag, void* stream) {
  if (dt != DET_F32 && dt != DET_BF16) return fail(DET_EDTYPE, "unknown dtype %d", static_cast<int>(dt));
  if (rows < 0 || cols < 0 || s_row < 0 || s_col < 0) return fail(DET_EINVAL, "negative size or stride");
  if (rows == 0 || cols == 0) return DET_OK;
  if (p == nullptr || flag == nullptr) return fail(DET_EINVAL, "null pointer");
  const dim3 grid(grid_for(rows * cols, 256, 4096));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == DET_F32) hipLaunchKernelGGL(k_check_finite<DET_F32>, grid, dim3(256), 0, s, p, rows, cols, s_row, s_col, flag);
  else hipLaunchKernelGGL(k_check_finite<DET_BF16>, grid, dim3(256), 0, s, p, rows, cols, s_row, s_col, flag);
  return hip_check(hipGetLastError(), "check_finite launch");
}

}  // extern "C"
