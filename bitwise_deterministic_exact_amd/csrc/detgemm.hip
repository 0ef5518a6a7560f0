// Exact long-accumulator GEMM for MI355X (gfx950): kernels and the C ABI.
//
// Follows the det-train page: "Method" (exact products, base-2^32 limbs added
// into signed int64 digits of a Kulisch accumulator, one rounding to fp32),
// "Usage" (det_gemm / det_gemm_partial / det_combine / det_finalize on x[M,K]
// and w[N,K] and their K-slices) and "Requirements and limits" (K <= 2^19,
// bf16 and f32).  The accumulator layout and rounding are documented in
// include/detgemm.h.
//
// The accumulate step is exact integer work, so it runs on the vector and
// scalar ALUs and the LDS, not on the matrix cores; the GEMM kernel below
// describes the work split and the accumulator.  The epilogue either writes
// the raw digits or rounds them in registers to fp32.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "detgemm.h"

namespace {

constexpr int ND = DET_NUM_DIGITS;   // 18 digits per output
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

// Packed exponent word (see decode below): the exponent offset sits at bits
// 5..14 and, for raw digits, the sign at bit 15.
constexpr uint32_t EXP_SHIFT = 5;
constexpr uint32_t SIGN_BIT = 15;

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
//
// Work split.  Every workgroup is a single wave that owns a 2 x 64 block of
// outputs: rows m0 and m0+1, lane l owning column n0+l of both.  There is no
// cross-wave sharing and so no barrier anywhere in the main loop.  Per 16-wide
// K-chunk:
//   * each lane loads its column's 16 raw w elements straight into registers
//     (vector loads issued one chunk ahead, so their latency hides behind the
//     current chunk; they are tracked by vmcnt, independent of the LDS
//     atomics);
//   * lane l loads and decodes x element k0 + (l mod 16) of both rows, so each
//     16-lane row of the wave holds the chunk's x values; the operand for step
//     j is broadcast to the whole wave with a DPP row broadcast of lane j;
//   * each lane decodes its w element once per k and uses it for both rows.
//
// Accumulator.  Each output owns 35 signed 32-bit counters in LDS, one per
// 16-bit field of the digit array (field q weighs 2^(16q - 298); digit
// j = field 2j + 2^16 * field 2j+1; products never reach bits >= 2^554, so
// field 35 would always be zero).  A product at bit offset o = ex + ew + 298
// is shifted by o mod 16 into a 64-bit T (|T| < 2^63) whose four 16-bit
// fields are added, each with one ds_add_u32, into counters o/16 .. o/16+3
// (bf16: |T| < 2^31, two fields).  The LDS address is the only per-lane
// dynamic index the hardware has, and a 32-bit atomic carrying a 16-bit field
// costs less LDS time per product than 64-bit limb atomics.  A field is below
// 2^16 in magnitude, so a counter takes 2^15 adds; every 2^15 k the counters
// are folded into int64 digits held in registers.
//
// Field conventions (template parameter TWOS):
//   false (det_gemm_partial): the fields of |product| each carry the product's
//     sign, so digit j is exactly the raw digit of the definition, the sum
//     over products of sign * bits [32j, 32j+32) of |p| * 2^298.
//   true (det_gemm): the fields of the signed product in two's complement (top
//     field signed).  Each product's fields still add up to its exact value,
//     so the digit array holds the same exact sum and rounds to the same fp32,
//     with fewer instructions per product.
//
// Counter layout: byte address field*512 + row*256 + lane*4, so the 64 lanes
// always hit 64 distinct banks whatever their fields.

constexpr int V_BN = 64;                    // columns per wave (one per lane)
constexpr int V_KC = 16;                    // K per chunk
constexpr int NF = 35;                      // 16-bit fields per output
constexpr int ROW_BYTES = 64 * 4;           // counters of one row: 64 lanes x 4 bytes
constexpr int64_t KFLUSH = int64_t(1) << 15;      // adds a counter can take

struct GemmArgs {
  const void* x; int64_t x_sm, x_sk;
  const void* w; int64_t w_sn, w_sk;
  int64_t M, N, K;
  int64_t tiles_m, tiles_n;
  int w_vec;                          // w rows contiguous and 16-byte aligned per chunk
  const int32_t* wsig;                // pre-decoded w (workspace): significands [Kp/16][Np][16]
  const uint16_t* wexp;               // pre-decoded w: exponent words [Kp/16][Np][16]
  int64_t wld;                        // Np * 16, the chunk pitch of both
  int64_t* acc;                       // digits [M][N][18]: the partial's output, or scratch
  float* y; int64_t y_sm, y_sn;       // gemm: fp32 out
  int epi;                            // epilogue, see EPI_* below
};

// Operand decode: value = (signed) m * 2^(exponent - bias).  SIDE 0 is x, 1
// is w; the exponent offsets are split between the sides so that, with
// sum = e_x + e_w, bits 5..14 of sum hold the product's bit offset
// o = ex + ew + 298 (f32: max(Ex,1) + max(Ew,1) - 2, bf16: max(Ex,1) +
// max(Ew,1) + 30).  The shift by 5 lets one bit-field extract give the shift
// inside a 16-bit field (bits 5..8) and one mask give the field's counter
// offset (bits 9..14).  With TWOS the sign is applied to m (two's
// complement); otherwise m is the magnitude and the sign sits in bit 15, so
// bit 15 of sum is the product's sign.  Subnormals keep their raw fraction
// and exponent 1: nothing is flushed.  For every bit pattern o <= 540, so no
// field index leaves 0..34.
template <int DT, bool TWOS, int SIDE, uint32_t ESH = EXP_SHIFT>
__device__ __forceinline__ void decode(uint32_t b, int32_t& m, uint32_t& e) {
  uint32_t E, mag, neg;
  if (DT == DET_F32) {
    E = (b >> 23) & 0xFFu;
    mag = (b & 0x7FFFFFu) | (min(E, 1u) << 23);
    neg = b >> 31;
  } else {
    E = (b >> 7) & 0xFFu;
    mag = (b & 0x7Fu) | (min(E, 1u) << 7);
    neg = (b >> 15) & 1u;
  }
  const uint32_t off = SIDE == 1 ? 0u : (DT == DET_F32 ? static_cast<uint32_t>(-2) : 30u);
  if (TWOS) {
    const uint32_t sgn = 0u - neg;
    m = static_cast<int32_t>((mag ^ sgn) + neg);
    e = (max(E, 1u) + off) << ESH;
  } else {
    m = static_cast<int32_t>(mag);
    e = ((max(E, 1u) + off) << ESH) + (neg << SIGN_BIT);
  }
}

// one exact product into the counters of one output; `sum` = e_x + e_w.
// Counter byte address: field*(R*256) + row*256 + lane*4.
template <int DT, bool TWOS, int R>
__device__ __forceinline__ void accumulate(char* lane_row, int32_t xm, int32_t wm, uint32_t sum) {
  constexpr int F = R * ROW_BYTES / 4;                  // ints between fields
  const uint32_t s16 = (sum >> EXP_SHIFT) & 15u;        // shift inside the field
  int* p = reinterpret_cast<int*>(lane_row + ((sum >> (EXP_SHIFT + 4)) & 63u) * (R * ROW_BYTES));   // field o/16
  if (DT == DET_F32) {
    uint64_t T;
    if (TWOS) T = static_cast<uint64_t>(static_cast<int64_t>(xm) * wm) << s16;
    else T = (static_cast<uint64_t>(static_cast<uint32_t>(xm)) * static_cast<uint32_t>(wm)) << s16;
    const uint32_t lo = static_cast<uint32_t>(T), hi = static_cast<uint32_t>(T >> 32);
    if (TWOS) {
      atomicAdd(p, static_cast<int>(lo & 0xFFFFu));
      atomicAdd(p + F, static_cast<int>(lo >> 16));
      atomicAdd(p + 2 * F, static_cast<int>(hi & 0xFFFFu));
      atomicAdd(p + 3 * F, static_cast<int>(hi) >> 16);
    } else {
      const uint32_t neg = (sum >> SIGN_BIT) & 1u, msk = 0u - neg;   // (f ^ msk) + neg = +-f
      atomicAdd(p, static_cast<int>(((lo & 0xFFFFu) ^ msk) + neg));
      atomicAdd(p + F, static_cast<int>(((lo >> 16) ^ msk) + neg));
      atomicAdd(p + 2 * F, static_cast<int>(((hi & 0xFFFFu) ^ msk) + neg));
      atomicAdd(p + 3 * F, static_cast<int>(((hi >> 16) ^ msk) + neg));
    }
  } else {
    if (TWOS) {
      const int32_t T = (xm * wm) << s16;               // |T| < 2^31
      atomicAdd(p, T & 0xFFFF);
      atomicAdd(p + F, T >> 16);
    } else {
      const uint32_t T = (static_cast<uint32_t>(xm) * static_cast<uint32_t>(wm)) << s16;
      const uint32_t neg = (sum >> SIGN_BIT) & 1u, msk = 0u - neg;
      atomicAdd(p, static_cast<int>(((T & 0xFFFFu) ^ msk) + neg));
      atomicAdd(p + F, static_cast<int>(((T >> 16) ^ msk) + neg));
    }
  }
}

// 24-bit field grid, used by det_gemm on f32 (two's-complement fields):
// counter p weighs 2^(24p - 298).  A product at offset o (plain, not shifted)
// goes to p = o div 24 with shift s = o mod 24; its value T = P * 2^s (P the
// signed significand product, |P| < 2^48, so |T| < 2^71) splits into fields
// g0 = bits 0..23 and g1 = bits 24..47 (both >= 0) and the signed
// g2 = T >> 48.  Three atomics per product instead of four; a counter takes
// 128 adds (|field| < 2^24) before it must be folded.
constexpr int NF24 = 24;                    // 24 x 24 = 576 bits
constexpr int64_t KFLUSH24 = 128;

template <int R>
__device__ __forceinline__ void accumulate24(char* lane_row, int32_t xm, int32_t wm, uint32_t o) {
  constexpr int F = R * ROW_BYTES / 4;
  const uint32_t p = __umulhi(o, 178956971u);           // o div 24 (exact for o < 2^30)
  const uint32_t s = o - 24u * p;
  int* ptr = reinterpret_cast<int*>(lane_row + p * (R * ROW_BYTES));
  const int64_t P = static_cast<int64_t>(xm) * wm;
  const uint64_t T = static_cast<uint64_t>(P) << s;     // bits 0..63 of P * 2^s
  const uint32_t lo = static_cast<uint32_t>(T), hi = static_cast<uint32_t>(T >> 32);
  atomicAdd(ptr, static_cast<int>(lo & 0xFFFFFFu));
  atomicAdd(ptr + F, static_cast<int>(__builtin_amdgcn_perm(hi, lo, 0x0C050403u)));   // bits 24..47
  atomicAdd(ptr + 2 * F, static_cast<int>(static_cast<uint64_t>(P >> (48u - s))));    // bits 48..71
}

// fold the 24 counters of one row into int64 digits (counter p lands at bit
// 24p = 32*(p*3/4) + 8*(3p mod 4)) and clear them; every `norm` folds, carry
// the digits so that all but the top one lie in [0, 2^32)
template <int R>
__device__ __forceinline__ void fold_row24(char* lane_row, int64_t (&dg)[ND], bool norm) {
  int* c = reinterpret_cast<int*>(lane_row);
  constexpr int F = R * ROW_BYTES / 4;
#pragma unroll
  for (int p = 0; p < NF24; ++p) {
    const int bit = 24 * p;
    dg[bit >> 5] += static_cast<int64_t>(c[p * F]) * (int64_t(1) << (bit & 31));
    c[p * F] = 0;
  }
  if (norm) {
#pragma unroll
    for (int j = 0; j + 1 < ND; ++j) {
      const int64_t carry = dg[j] >> 32;
      dg[j] -= carry * (int64_t(1) << 32);
      dg[j + 1] += carry;
    }
  }
}

template <int DT>
__device__ __forceinline__ uint32_t load_elem(const void* base, int64_t idx) {
  return DT == DET_F32 ? static_cast<const uint32_t*>(base)[idx]
                       : static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]);
}

// the lane's 16 raw w elements of chunk k0 (zero beyond K or beyond N)
template <int DT>
__device__ __forceinline__ void load_w_chunk(const GemmArgs& a, const void* __restrict__ wg, int64_t wrow,
                                             bool n_ok, int64_t k0, uint32_t (&wr)[V_KC]) {
  if (a.w_vec && k0 + V_KC <= a.K) {
    if (DT == DET_F32) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(wg) + wrow + k0);
#pragma unroll
      for (int i = 0; i < V_KC / 4; ++i) {
        const uint4 v = p[i];
        wr[4 * i] = v.x; wr[4 * i + 1] = v.y; wr[4 * i + 2] = v.z; wr[4 * i + 3] = v.w;
      }
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(wg) + wrow + k0);
#pragma unroll
      for (int i = 0; i < V_KC / 8; ++i) {
        const uint4 v = p[i];
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) { wr[8 * i + 2 * t] = q[t] & 0xFFFFu; wr[8 * i + 2 * t + 1] = q[t] >> 16; }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < V_KC; ++i) {
      const int64_t k = min<int64_t>(k0 + i, a.K - 1);
      wr[i] = load_elem<DT>(wg, wrow + k * a.w_sk);
    }
  }
  if (!n_ok) {
#pragma unroll
    for (int i = 0; i < V_KC; ++i) wr[i] = 0u;
  }
  if (k0 + V_KC > a.K) {
#pragma unroll
    for (int i = 0; i < V_KC; ++i) wr[i] = (k0 + i < a.K) ? wr[i] : 0u;
  }
}

// fold the counters of one row into int64 digits and clear them
template <int R>
__device__ __forceinline__ void fold_row(char* lane_row, int64_t (&dg)[ND]) {
  int* c = reinterpret_cast<int*>(lane_row);
  constexpr int F = R * ROW_BYTES / 4;
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    const int hi = 2 * j + 1 < NF ? c[(2 * j + 1) * F] : 0;
    dg[j] += static_cast<int64_t>(c[(2 * j) * F]) + (static_cast<int64_t>(hi) << 16);
    c[(2 * j) * F] = 0;
    if (2 * j + 1 < NF) c[(2 * j + 1) * F] = 0;
  }
}

template <int J>
__device__ __forceinline__ int bcast(int v) {     // lane J of each 16-lane row, to the whole row
  return __builtin_amdgcn_mov_dpp(v, 0x150 + J, 0xF, 0xF, true);
}

// One K-chunk: step J uses w element J of the lane (raw bits to decode, or,
// with PRE, a pre-decoded significand and the packed exponent words) and
// broadcasts x element J of each row from lane J of every 16-lane row.
template <int DT, bool TWOS, int R, bool PRE, bool G24, int J>
__device__ __forceinline__ void steps(char* lane_base, const uint32_t (&wa)[V_KC], const uint32_t (&wb)[V_KC / 2],
                                      const int (&xm)[R], const int (&xe)[R]) {
  int32_t wm;
  uint32_t we;
  if (PRE) {
    wm = static_cast<int32_t>(wa[J]);
    we = (J & 1) ? (wb[J / 2] >> 16) : (wb[J / 2] & 0xFFFFu);
  } else {
    decode<DT, TWOS, 1, G24 ? 0u : EXP_SHIFT>(wa[J], wm, we);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t sum = static_cast<uint32_t>(bcast<J>(xe[r])) + we;
    if (G24) accumulate24<R>(lane_base + r * ROW_BYTES, bcast<J>(xm[r]), wm, sum);
    else accumulate<DT, TWOS, R>(lane_base + r * ROW_BYTES, bcast<J>(xm[r]), wm, sum);
  }
  if constexpr (J + 1 < V_KC) steps<DT, TWOS, R, PRE, G24, J + 1>(lane_base, wa, wb, xm, xe);
}

// the lane's pre-decoded w chunk: 16 significands and 16 exponent words
// (rows padded to the tile and K to the chunk, so no bounds logic).  The
// workspace is chunk-major, so a wave's 64 lanes read one contiguous 4 KiB
// of significands and 2 KiB of exponents, whatever the length of K.
__device__ __forceinline__ void load_w_pre(const GemmArgs& a, int64_t n, int64_t k0, uint32_t (&wa)[V_KC],
                                           uint32_t (&wb)[V_KC / 2]) {
  const int64_t off = (k0 / V_KC) * a.wld + n * V_KC;
  const uint4* ps = reinterpret_cast<const uint4*>(a.wsig + off);
  const uint4* pe = reinterpret_cast<const uint4*>(a.wexp + off);
#pragma unroll
  for (int i = 0; i < V_KC / 4; ++i) {
    const uint4 v = ps[i];
    wa[4 * i] = v.x; wa[4 * i + 1] = v.y; wa[4 * i + 2] = v.z; wa[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < V_KC / 8; ++i) {
    const uint4 v = pe[i];
    wb[4 * i] = v.x; wb[4 * i + 1] = v.y; wb[4 * i + 2] = v.z; wb[4 * i + 3] = v.w;
  }
}

// R rows per wave.  TWOS = false: write raw digits; TWOS = true: round to fp32.
// Epilogues.  A K range longer than one block is run as several launches
// that carry the exact digits from one to the next (see launch_gemm_rows).
constexpr int EPI_ROUND = 0;        // round the digits to fp32 into y
constexpr int EPI_STORE = 1;        // write the digits to acc
constexpr int EPI_ADD = 2;          // add acc's digits, write them back
constexpr int EPI_ADD_ROUND = 3;    // add acc's digits, round to fp32 into y

// R rows per wave; PRE: w comes pre-decoded from the workspace; G24: the
// 24-bit field grid (f32 with TWOS only), else 16-bit fields.
template <int DT, bool TWOS, int R, bool PRE, bool G24>
__global__ __launch_bounds__(64) void k_gemm(GemmArgs a, const void* __restrict__ xg,
                                             const void* __restrict__ wg) {
  static_assert(!G24 || (DT == DET_F32 && TWOS), "the 24-bit grid serves f32 det_gemm only");
  constexpr int NFG = G24 ? NF24 : NF;
  constexpr int64_t KF = G24 ? KFLUSH24 : KFLUSH;
  __shared__ __align__(16) int counters[NFG * R * 64];

  const int lane = threadIdx.x;
  // Workgroups are dispatched to the 8 XCDs round-robin, each XCD with its
  // own L2.  Give every XCD a contiguous range of tiles in column-major tile
  // order, so the waves resident on one XCD share one 64-column slice of w
  // (kept in that L2) while they walk down the rows.
  const int64_t nb = gridDim.x, b = blockIdx.x;
  const int64_t xcd = b % 8, per = nb / 8, extra = nb % 8;
  const int64_t tile = xcd * per + min(xcd, extra) + b / 8;
  const int64_t tn = tile / a.tiles_m, tm = tile % a.tiles_m;
  const int64_t m0 = tm * R, n0 = tn * V_BN;
  char* const lane_base = reinterpret_cast<char*>(counters) + lane * 4;

#pragma unroll
  for (int q = 0; q < NFG * R; ++q) counters[q * 64 + lane] = 0;

  const int64_t n = n0 + lane;
  const bool n_ok = n < a.N;
  const int64_t wrow = (n_ok ? n : a.N - 1) * a.w_sn;
  bool row_ok[R];
  int64_t xrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    row_ok[r] = m0 + r < a.M;
    xrow[r] = min(m0 + r, a.M - 1) * a.x_sm;
  }
  const int xj = lane & 15;                       // this lane's k within a chunk (x side)

  int64_t dg[R][ND];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < ND; ++j) dg[r][j] = 0;

  // chunk 0 operands
  uint32_t wnext[V_KC], wbnext[V_KC / 2];
#pragma unroll
  for (int i = 0; i < V_KC / 2; ++i) wbnext[i] = 0u;
  uint32_t xn[R];
#pragma unroll
  for (int r = 0; r < R; ++r) xn[r] = 0u;
  if (a.K > 0) {
    if (PRE) load_w_pre(a, n, 0, wnext, wbnext);
    else load_w_chunk<DT>(a, wg, wrow, n_ok, 0, wnext);
    const int64_t k = min<int64_t>(xj, a.K - 1);
#pragma unroll
    for (int r = 0; r < R; ++r) xn[r] = load_elem<DT>(xg, xrow[r] + k * a.x_sk);
  }

  for (int64_t k0 = 0; k0 < a.K; k0 += V_KC) {
    uint32_t wr[V_KC], wb[V_KC / 2];
#pragma unroll
    for (int i = 0; i < V_KC; ++i) wr[i] = wnext[i];
#pragma unroll
    for (int i = 0; i < V_KC / 2; ++i) wb[i] = wbnext[i];
    const bool kin = k0 + xj < a.K;
    int xm[R], xe[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int32_t m;
      uint32_t e;
      decode<DT, TWOS, 0, G24 ? 0u : EXP_SHIFT>((row_ok[r] && kin) ? xn[r] : 0u, m, e);
      xm[r] = m;
      xe[r] = static_cast<int>(e);
    }
    if (k0 + V_KC < a.K) {                        // prefetch the next chunk
      if (PRE) load_w_pre(a, n, k0 + V_KC, wnext, wbnext);
      else load_w_chunk<DT>(a, wg, wrow, n_ok, k0 + V_KC, wnext);
      const int64_t k = min<int64_t>(k0 + V_KC + xj, a.K - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) xn[r] = load_elem<DT>(xg, xrow[r] + k * a.x_sk);
    }
    steps<DT, TWOS, R, PRE, G24, 0>(lane_base, wr, wb, xm, xe);
    if (a.K > KF && ((k0 + V_KC) % KF) == 0) {    // counters near their limit
      // (24-bit grid: carry the digits every 16 folds, 2^56 growth per fold)
      const bool norm = ((k0 + V_KC) % (16 * KF)) == 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (G24) fold_row24<R>(lane_base + r * ROW_BYTES, dg[r], norm);
        else fold_row<R>(lane_base + r * ROW_BYTES, dg[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (G24) fold_row24<R>(lane_base + r * ROW_BYTES, dg[r], true);
    else fold_row<R>(lane_base + r * ROW_BYTES, dg[r]);
  }

  if (!n_ok) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t m = m0 + r;
    if (m >= a.M) continue;
    int64_t* d = a.acc + (m * a.N + n) * ND;
    if (a.epi == EPI_ADD || a.epi == EPI_ADD_ROUND) {
#pragma unroll
      for (int j = 0; j < ND; ++j) dg[r][j] += d[j];
    }
    if (a.epi == EPI_STORE || a.epi == EPI_ADD) {
#pragma unroll
      for (int j = 0; j < ND; ++j) d[j] = dg[r][j];
    } else {
      a.y[m * a.y_sm + n * a.y_sn] = __uint_as_float(round_digits_to_f32(dg[r]));
    }
  }
}

// ---------------------------------------------------------------- w pre-decode
// w [N][K] (any strides) -> significands int32 and exponent words uint16,
// both [Kp/16][Np][16] (chunk-major: the 16 k of one chunk of row n are
// contiguous, rows follow each other), zero outside N x K.  The GEMM kernel
// then loads w with aligned 16-byte loads, coalesced across the wave, and
// spends no instructions on decoding it.  (Row-major [Np][Kp] put each lane
// of a wave in its own 2 MiB page once K reached 2^19, and the GEMM ran at
// half speed.)
struct PredecodeArgs {
  const void* w; int64_t w_sn, w_sk;
  int64_t N, K, Np, Kp;
  int32_t* wsig; uint16_t* wexp;
};

template <int DT, bool TWOS, uint32_t ESH>
__global__ __launch_bounds__(256) void k_predecode_w(PredecodeArgs a) {
  const int64_t total = a.Np * a.Kp;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t c = i / (a.Np * V_KC), r = i % (a.Np * V_KC);
    const int64_t n = r / V_KC, k = c * V_KC + r % V_KC;
    int32_t m = 0;
    uint32_t e = 0u;
    if (n < a.N && k < a.K) decode<DT, TWOS, 1, ESH>(load_elem<DT>(a.w, n * a.w_sn + k * a.w_sk), m, e);
    a.wsig[i] = m;
    a.wexp[i] = static_cast<uint16_t>(e);
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

unsigned grid_for(int64_t n, int64_t per_block, unsigned cap) {
  int64_t g = (n + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return static_cast<unsigned>(g > cap ? cap : g);
}

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// K per launch.  With a longer K range the waves resident on one XCD drift
// apart in k and stop sharing their slice of w in L2 (measured: 2400 GMAC/s at
// K = 2^15, 824 at K = 2^19 in one launch), so longer ranges run as several
// launches of this length that carry the exact digits between them.
constexpr int64_t K_BLOCK = int64_t(1) << 15;

// workspace: the pre-decoded w, then (det_gemm with K > K_BLOCK) int64
// digit scratch for the output
int64_t predecode_bytes(int64_t N, int64_t K) { return round_up(N, V_BN) * round_up(K, V_KC) * (4 + 2); }
int64_t workspace_bytes(int out_mode, int64_t M, int64_t N, int64_t K) {
  int64_t b = predecode_bytes(N, K);
  if (out_mode == 1 && K > K_BLOCK) b += M * N * ND * 8;
  return b;
}

template <int R>
det_status launch_gemm_rows(det_dtype dt, int out_mode, GemmArgs a, void* ws, hipStream_t s) {
  a.tiles_m = (a.M + R - 1) / R;
  a.tiles_n = (a.N + V_BN - 1) / V_BN;
  const int64_t blocks = a.tiles_m * a.tiles_n;
  if (blocks == 0) return DET_OK;
  if (blocks > 0x7FFFFFFF) return fail(DET_EINVAL, "too many output tiles");
  // 16-byte vector loads of w chunks: unit K-stride and every chunk start aligned
  const int64_t esz = dt == DET_F32 ? 4 : 2;
  a.w_vec = a.w_sk == 1 && (reinterpret_cast<uintptr_t>(a.w) % 16) == 0 && (a.w_sn * esz) % 16 == 0;
  const bool pre = ws != nullptr && a.K > 0;
  if (pre) {
    PredecodeArgs p{};
    p.w = a.w; p.w_sn = a.w_sn; p.w_sk = a.w_sk;
    p.N = a.N; p.K = a.K; p.Np = round_up(a.N, V_BN); p.Kp = round_up(a.K, V_KC);
    p.wsig = static_cast<int32_t*>(ws);
    p.wexp = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + p.Np * p.Kp * 4);
    a.wsig = p.wsig; a.wexp = p.wexp; a.wld = p.Np * V_KC;
    const dim3 pg(grid_for(p.Np * p.Kp, 256, 8192));
    if (dt == DET_F32) {
      if (out_mode == 0) hipLaunchKernelGGL((k_predecode_w<DET_F32, false, EXP_SHIFT>), pg, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((k_predecode_w<DET_F32, true, 0>), pg, dim3(256), 0, s, p);
    } else {
      if (out_mode == 0) hipLaunchKernelGGL((k_predecode_w<DET_BF16, false, EXP_SHIFT>), pg, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((k_predecode_w<DET_BF16, true, EXP_SHIFT>), pg, dim3(256), 0, s, p);
    }
    det_status st = hip_check(hipGetLastError(), "predecode launch");
    if (st != DET_OK) return st;
  }
  const dim3 grid(static_cast<unsigned>(blocks)), block(64);
#define DET_LAUNCH(DTV, TW, PR, G) hipLaunchKernelGGL((k_gemm<DTV, TW, R, PR, G>), grid, block, 0, s, b, xb, a.w)
  // K blocks (one block without a workspace, or when K is short)
  const int64_t kblk = pre ? K_BLOCK : a.K;
  const int64_t nblk = a.K > 0 ? (a.K + kblk - 1) / kblk : 1;
  const int64_t esx = dt == DET_F32 ? 4 : 2;
  if (out_mode == 1 && nblk > 1)                  // digit scratch behind the decoded w
    a.acc = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + predecode_bytes(a.N, a.K));
  for (int64_t ib = 0; ib < nblk; ++ib) {
    GemmArgs b = a;
    const int64_t k0 = ib * kblk;
    b.K = min(kblk, a.K - k0);
    const void* xb = static_cast<const char*>(a.x) + k0 * a.x_sk * esx;
    if (pre) { b.wsig = a.wsig + k0 / V_KC * a.wld; b.wexp = a.wexp + k0 / V_KC * a.wld; }
    const bool first = ib == 0, last = ib + 1 == nblk;
    if (out_mode == 0) b.epi = first ? EPI_STORE : EPI_ADD;
    else b.epi = nblk == 1 ? EPI_ROUND : first ? EPI_STORE : last ? EPI_ADD_ROUND : EPI_ADD;
    if (dt == DET_F32) {
      if (out_mode == 0) { if (pre) DET_LAUNCH(DET_F32, false, true, false); else DET_LAUNCH(DET_F32, false, false, false); }
      else { if (pre) DET_LAUNCH(DET_F32, true, true, true); else DET_LAUNCH(DET_F32, true, false, true); }
    } else {
      if (out_mode == 0) { if (pre) DET_LAUNCH(DET_BF16, false, true, false); else DET_LAUNCH(DET_BF16, false, false, false); }
      else { if (pre) DET_LAUNCH(DET_BF16, true, true, false); else DET_LAUNCH(DET_BF16, true, false, false); }
    }
    det_status st = hip_check(hipGetLastError(), "gemm launch");
    if (st != DET_OK) return st;
  }
#undef DET_LAUNCH
  return DET_OK;
}

// Two rows per wave: the 17.9 KB of counters per wave let 8-9 waves share a
// CU; four rows (one wave per SIMD) measured 40% slower on MI355X.
det_status launch_gemm(det_dtype dt, int out_mode, GemmArgs a, void* ws, hipStream_t s) {
  return launch_gemm_rows<2>(dt, out_mode, a, ws, s);
}

}  // namespace

// ---------------------------------------------------------------- C ABI
extern "C" {

int det_num_digits(void) { return ND; }
int det_lsb_exponent(void) { return DET_LSB_EXPONENT; }
int64_t det_k_max(void) { return DET_K_MAX; }
const char* det_last_error(void) { return g_err; }

namespace {

det_status gemm_common(int out_mode, det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk, const void* w,
                       int64_t w_sn, int64_t w_sk, int64_t M, int64_t N, int64_t K, float* y, int64_t y_sm,
                       int64_t y_sn, int64_t* acc, void* ws, size_t ws_bytes, void* stream) {
  det_status st = check_operands(dt, x, x_sm, x_sk, w, w_sn, w_sk, M, N, K);
  if (st != DET_OK) return st;
  if (out_mode == 1) {
    if (M > 0 && N > 0 && y == nullptr) return fail(DET_EINVAL, "null output");
    if (y_sm < 0 || y_sn < 0) return fail(DET_EINVAL, "negative output stride");
    if (reinterpret_cast<uintptr_t>(y) & 3u) return fail(DET_EINVAL, "output must be 4-byte aligned");
  } else {
    if (M > 0 && N > 0 && acc == nullptr) return fail(DET_EINVAL, "null accumulator");
    if (reinterpret_cast<uintptr_t>(acc) & 7u) return fail(DET_EINVAL, "accumulator must be 8-byte aligned");
  }
  if (ws != nullptr) {
    if (reinterpret_cast<uintptr_t>(ws) & 15u) return fail(DET_EINVAL, "workspace must be 16-byte aligned");
    if (ws_bytes < static_cast<size_t>(workspace_bytes(out_mode, M, N, K)))
      return fail(DET_EINVAL, "workspace of %zu bytes is smaller than the %lld needed", ws_bytes,
                  (long long)workspace_bytes(out_mode, M, N, K));
  }
  GemmArgs a{};
  a.x = x; a.x_sm = x_sm; a.x_sk = x_sk;
  a.w = w; a.w_sn = w_sn; a.w_sk = w_sk;
  a.M = M; a.N = N; a.K = K;
  a.y = y; a.y_sm = y_sm; a.y_sn = y_sn;
  a.acc = acc;
  return launch_gemm(dt, out_mode, a, ws, static_cast<hipStream_t>(stream));
}

}  // namespace

int64_t det_gemm_workspace_bytes(det_dtype dt, int partial, int64_t M, int64_t N, int64_t K) {
  (void)dt;
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return workspace_bytes(partial ? 0 : 1, M, N, K);
}

det_status det_gemm(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk, const void* w, int64_t w_sn,
                    int64_t w_sk, int64_t M, int64_t N, int64_t K, float* y, int64_t y_sm, int64_t y_sn,
                    void* stream) {
  return gemm_common(1, dt, x, x_sm, x_sk, w, w_sn, w_sk, M, N, K, y, y_sm, y_sn, nullptr, nullptr, 0, stream);
}

det_status det_gemm_ws(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk, const void* w, int64_t w_sn,
                       int64_t w_sk, int64_t M, int64_t N, int64_t K, float* y, int64_t y_sm, int64_t y_sn,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr && M > 0 && N > 0 && K > 0) return fail(DET_EINVAL, "null workspace");
  return gemm_common(1, dt, x, x_sm, x_sk, w, w_sn, w_sk, M, N, K, y, y_sm, y_sn, nullptr, workspace,
                     workspace_bytes, stream);
}

det_status det_gemm_partial(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk, const void* w,
                            int64_t w_sn, int64_t w_sk, int64_t M, int64_t N, int64_t K, int64_t* acc,
                            void* stream) {
  return gemm_common(0, dt, x, x_sm, x_sk, w, w_sn, w_sk, M, N, K, nullptr, 0, 0, acc, nullptr, 0, stream);
}

det_status det_gemm_partial_ws(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk, const void* w,
                               int64_t w_sn, int64_t w_sk, int64_t M, int64_t N, int64_t K, int64_t* acc,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr && M > 0 && N > 0 && K > 0) return fail(DET_EINVAL, "null workspace");
  return gemm_common(0, dt, x, x_sm, x_sk, w, w_sn, w_sk, M, N, K, nullptr, 0, 0, acc, workspace,
                     workspace_bytes, stream);
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
