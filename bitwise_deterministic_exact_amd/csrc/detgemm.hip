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

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

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

// Optional timing of a call's main GEMM kernel (det_set_kernel_events): the
// calling thread's two events, recorded on the call's stream just before the
// first and just after the last launch of the kernel that forms the call's
// products (k_gemm8, k_slice_mma or k_partial).  Null: nothing is recorded.
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

det_status mark_event(hipEvent_t ev, bool now, hipStream_t s) {
  if (!now || ev == nullptr) return DET_OK;
  return hip_check(hipEventRecord(ev, s), "kernel timing event");
}
// which of the two events a launcher records (several launchers in one call
// share the interval: the first records the start, the last the stop)
constexpr int MARK_START = 1, MARK_STOP = 2, MARK_BOTH = 3;

// Conditions only the kernels can see, kept per GPU until cleared (sticky,
// like IEEE 754's exception flags): word 0 becomes 1 when an operand element
// is Inf or NaN, word 1 when a digit handed to combine or finalize, or a
// digit sum of combine, lies outside +-2^62.  Kernels store 1 and never 0;
// only det_device_status clears the words.  In host code the array's name is
// a host-side stand-in: host code uses the address status_words() looks up.
static __device__ __align__(16) int32_t g_dev_status[4];

template <int DT>
__device__ __forceinline__ bool nonfinite_bits(uint32_t b) {
  return DT == DET_F32 ? (b & 0x7F800000u) == 0x7F800000u : (b & 0x7F80u) == 0x7F80u;
}
__device__ __forceinline__ void note_nonfinite(bool bad) {
  if (bad) g_dev_status[0] = 1;
}
__device__ __forceinline__ bool digit_in_range(int64_t v) {        // -2^62 <= v <= 2^62
  return static_cast<uint64_t>(v) + (uint64_t(1) << 62) <= (uint64_t(1) << 63);
}
__device__ __forceinline__ void note_range(bool bad) {
  if (bad) g_dev_status[1] = 1;
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
//
// round_words_to_f32: the same value after the carries have been propagated,
// (W + carry * 2^576) * 2^-298 with W = sum w[j] 2^(32j), 0 <= w[j] < 2^32.
__device__ uint32_t round_words_to_f32(uint32_t (&w)[ND], int64_t carry) {
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

// round_digits_to_f32: the carries of the digits, then the rounding
__device__ uint32_t round_digits_to_f32(const int64_t (&dg)[ND]) {
  uint32_t w[ND];
  int64_t carry = 0;
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    const int64_t t = dg[j] + carry;
    w[j] = static_cast<uint32_t>(t);
    carry = t >> 32;                  // arithmetic: floor(t / 2^32)
  }
  return round_words_to_f32(w, carry);
}

// ---------------------------------------------------------------- GEMM kernels: shared parts
//
// Both GEMM kernels give lane l of a wave column n0 + l of a 64-column output
// tile and walk K in 16-wide chunks.  Per chunk:
//   * each lane loads its column's 16 w elements straight into registers
//     (vector loads issued one chunk ahead, so their latency hides behind the
//     current chunk; they are tracked by vmcnt, independent of the LDS
//     atomics), either raw or pre-decoded from a workspace;
//   * lane l loads and decodes x element k0 + (l mod 16) of each of its rows,
//     so each 16-lane row of the wave holds the chunk's x values; the operand
//     for step j is broadcast to the whole wave with a DPP row broadcast of
//     lane j;
//   * each lane uses its w element once per row.
// The exact products are accumulated in LDS with integer atomics whose
// address depends on the product's exponent: the LDS address is the only
// per-lane dynamic index the hardware has.  k_gemm (the raw digits of
// det_gemm_partial) and k_gemm8 (det_gemm) differ in what they add where.

constexpr int V_BN = 64;                    // columns per wave (one per lane)
constexpr int V_KC = 16;                    // K per chunk

struct GemmArgs {
  const void* x; int64_t x_sm, x_sk;
  const void* w; int64_t w_sn, w_sk;
  int64_t M, N, K;
  int64_t tiles_m, tiles_n;
  int w_vec;                          // w rows contiguous and 16-byte aligned per chunk
  const int32_t* wsig;                // pre-decoded w (workspace): significands [Kp/16][Np/64][4][64][4]
  const uint16_t* wexp;               // k_gemm: 16-bit exponent words [Kp/16][Np/64][2][64][8]
  const uint32_t* wexp32;             // k_gemm8: 32-bit words [Kp/16][Np/64][4][64][4]
  int64_t wld;                        // Np * 16, the chunk pitch of all three
  const int32_t* xsig;                // pre-decoded x of this K block: significands [Mp][xld]
  const uint32_t* xword;              // pre-decoded x: exponent / address words [Mp][xld]
  int64_t xld;                        // row pitch of both: the block's K padded to 16
  int64_t* acc;                       // digits [M][N][18]: the partial's output, or scratch
  float* y; int64_t y_sm, y_sn;       // gemm: fp32 out
  int epi;                            // epilogue, see EPI_* below
  // det_gemm on a subset (pre-decoded path only): row m of this GEMM is row
  // xmap[m] of x and of y, column n is row wmap[n] of w and column wmap[n]
  // of y; null maps are the identity
  const int32_t* xmap;
  const int32_t* wmap;
  // decided on the device (null: unused): the launch does nothing unless
  // *gate != 0; the listed form of k_gemm8 takes M from *mcount and N from
  // *ncount (M and N above are then their largest values)
  const int32_t* gate;
  const int32_t* mcount;
  const int32_t* ncount;
  int64_t tpw;                        // k_gemm8's looping form: consecutive tiles per workgroup
};

// Epilogues.  A K range longer than one block is run as several launches
// that carry the exact digits from one to the next (see the launchers).
constexpr int EPI_ROUND = 0;        // round the digits to fp32 into y
constexpr int EPI_STORE = 1;        // write the digits to acc
constexpr int EPI_ADD = 2;          // add acc's digits, write them back
constexpr int EPI_ADD_ROUND = 3;    // add acc's digits, round to fp32 into y

// Operand decode: value = (signed) m * 2^(exponent - bias).  SIDE 0 is x, 1
// is w; the exponent offsets are split between the sides so that the sum of
// the two exponent words is the product's bit offset o = ex + ew + 298
// (f32: max(Ex,1) + max(Ew,1) - 2, bf16: max(Ex,1) + max(Ew,1) + 30)
// shifted left by ESH, which each kernel picks so that its counter address
// and shift fall out of the sum with one or two bit operations.  With TWOS
// the sign is applied to m (two's complement); otherwise m is the magnitude
// and the sign sits in bit 15 (SIGN_BIT), so bit 15 of the sum is the
// product's sign.  Subnormals keep their raw fraction and exponent 1: nothing
// is flushed.  For every bit pattern o <= 540.
template <int DT, bool TWOS, int SIDE, uint32_t ESH>
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

template <int J>
__device__ __forceinline__ int bcast(int v) {     // lane J of each 16-lane row, to the whole row
  return __builtin_amdgcn_mov_dpp(v, 0x150 + J, 0xF, 0xF, true);
}

// Workgroups are dispatched to the 8 XCDs round-robin, each XCD with its own
// L2.  Give every XCD a contiguous range of tiles in column-major tile order,
// so the workgroups resident on one XCD share one 64-column slice of w (kept
// in that L2) while they walk down the rows.  xcd_tile_of(n): the same over
// the first n workgroups of a larger grid (blockIdx.x < n).
__device__ __forceinline__ int64_t xcd_tile_of(int64_t nb) {
  const int64_t b = blockIdx.x;
  const int64_t xcd = b % 8, per = nb / 8, extra = nb % 8;
  return xcd * per + min(xcd, extra) + b / 8;
}
__device__ __forceinline__ int64_t xcd_tile() { return xcd_tile_of(gridDim.x); }

// ---------------------------------------------------------------- raw-digit kernel (det_gemm_partial)
//
// The raw digits are per product and per 32-bit limb by definition (digit j
// = sum over products of sign * bits [32j, 32j+32) of |p| * 2^298), so the
// product is split at fixed 16-bit field boundaries: a product at bit offset
// o is shifted by o mod 16 into the 64-bit T = |P| * 2^(o mod 16) < 2^63,
// whose four 16-bit fields (bf16: T < 2^31, two fields) are added into
// counters o/16 .. o/16+3 with ds_add_u32 (for f32, two fields to one
// 64-bit counter with ds_add_u64: see steps_raw).  Digit j is then field 2j +
// 2^16 * field 2j+1.  Products with a negative sign go into a second set of
// counters (slots 64..98), so every add is an unsigned 16-bit field and
// the sign costs no instruction: digit j = (P[2j] - N[2j]) + 2^16 (P[2j+1] -
// N[2j+1]).
//
// Exponent words carry o << 5 and the sign at bit 15, so the sum of x's and
// w's words holds the shift inside a field at bits 5..8 and the slot (field
// + 64 * sign) at bits 9..15: the slot's byte offset is sum & 0xFE00 for a
// slot stride of 512 bytes (2 rows x 64 lanes x 4 bytes), one and-or with
// the lane's offset.  A counter takes 2^16 adds of a 16-bit field, and a
// launch covers at most 2^15 k, so there is nothing to fold before the end.
//
// The counters of a 2 x 64 tile fill 50 KB, shared, as in k_gemm8, by the W
// waves of a workgroup that take the K-chunks in turn; with no folds there
// is no barrier in the main loop.  At the end waves 0 and 1 turn their row's
// counters into digits.
constexpr int NF = 35;                      // 16-bit fields per output
constexpr int NEG_SLOT = 64;                // negative products' fields start here
constexpr int NSLOT = NEG_SLOT + NF;        // slots per output

// One chunk of the raw-digit kernel: step J, all rows.  PAIR: one row, and
// each slot holds 64-bit counters whose two 32-bit halves count two
// consecutive fields (slot f: field f low, field f + 1 high), so a product's
// four fields take two 64-bit atomics (bf16: two fields, one atomic).  A half
// takes at most 2^15 adds of a 16-bit field, so no carry crosses into the
// other half.
template <int DT, int R, bool PRE, bool PAIR, bool SX, int J>
__device__ __forceinline__ void steps_raw(char* cbase, uint32_t lane_off, const uint32_t (&wa)[V_KC],
                                          const uint32_t (&wb)[V_KC / 2], const int (&xm)[R], const int (&xe)[R],
                                          const uint32_t (&xs)[R][V_KC]) {
  static_assert(R * 64 * (PAIR ? 8 : 4) == 512, "slot offsets come from bits 9..15 of the exponent sum");
  int32_t wm;
  uint32_t we;
  if (PRE) {
    wm = static_cast<int32_t>(wa[J]);
    we = (J & 1) ? (wb[J / 2] >> 16) : (wb[J / 2] & 0xFFFFu);
  } else {
    decode<DT, false, 1, EXP_SHIFT>(wa[J], wm, we);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t sum = static_cast<uint32_t>(bcast<J>(xe[r])) + we;
    const uint32_t s16 = (sum >> EXP_SHIFT) & 15u;
    if constexpr (PAIR) {
      unsigned long long* const q = reinterpret_cast<unsigned long long*>(cbase + ((sum & 0xFE00u) | lane_off));
      constexpr int FQ = 512 / 8;               // counters between consecutive slots
      auto pair = [](uint32_t v) {
        return static_cast<unsigned long long>(v & 0xFFFFu) | (static_cast<unsigned long long>(v >> 16) << 32);
      };
      if (DT == DET_F32) {
        const uint32_t xv = SX ? xs[r][J] : static_cast<uint32_t>(bcast<J>(xm[r]));
        const uint64_t T = (static_cast<uint64_t>(xv) * static_cast<uint32_t>(wm)) << s16;
        // the halves as two opaque 32-bit values (an empty asm, no
        // instruction): each pair is then one and and one shift, where the
        // compiler otherwise rebuilds the fields with 64-bit shifts and moves
        uint32_t lo = static_cast<uint32_t>(T), hi = static_cast<uint32_t>(T >> 32);
        asm("" : "+v"(lo), "+v"(hi));
        atomicAdd(q, pair(lo));
        atomicAdd(q + 2 * FQ, pair(hi));
      } else {
        const uint32_t T = static_cast<uint32_t>(__umul24(static_cast<uint32_t>(bcast<J>(xm[r])),
                                                           static_cast<uint32_t>(wm))) << s16;
        atomicAdd(q, pair(T));
      }
      continue;
    }
    int* const p = reinterpret_cast<int*>(cbase + ((sum & 0xFE00u) | (lane_off + r * 256u)));
    constexpr int F = 512 / 4;                  // ints between consecutive fields
    if (DT == DET_F32) {
      const uint64_t T = (static_cast<uint64_t>(static_cast<uint32_t>(bcast<J>(xm[r]))) *
                          static_cast<uint32_t>(wm)) << s16;
      const uint32_t lo = static_cast<uint32_t>(T), hi = static_cast<uint32_t>(T >> 32);
      atomicAdd(p, static_cast<int>(lo & 0xFFFFu));
      atomicAdd(p + F, static_cast<int>(lo >> 16));
      atomicAdd(p + 2 * F, static_cast<int>(hi & 0xFFFFu));
      atomicAdd(p + 3 * F, static_cast<int>(hi >> 16));
    } else {
      const uint32_t T = static_cast<uint32_t>(__umul24(static_cast<uint32_t>(bcast<J>(xm[r])),
                                                         static_cast<uint32_t>(wm))) << s16;
      atomicAdd(p, static_cast<int>(T & 0xFFFFu));
      atomicAdd(p + F, static_cast<int>(T >> 16));
    }
  }
  if constexpr (J + 1 < V_KC) steps_raw<DT, R, PRE, PAIR, SX, J + 1>(cbase, lane_off, wa, wb, xm, xe, xs);
}

// the lane's pre-decoded w chunk: 16 significands and 16 exponent words
// (rows padded to the tile and K to the chunk, so no bounds logic).  Each
// chunk of the workspace holds, per 64-column tile, 16-byte sub-blocks laid
// out [4][64][4] for 32-bit words and [2][64][8] for 16-bit ones: every
// 16-byte load of the wave reads one contiguous 1 KiB, and the sub-blocks
// sit at fixed 1 KiB steps from the lane's pointer (immediate offsets).
// `ws`, `we` point at the lane's sub-block 0 of chunk 0.
__device__ __forceinline__ void load_w_pre(const GemmArgs& a, const int32_t* ws, const uint16_t* we, int64_t k0,
                                           uint32_t (&wa)[V_KC], uint32_t (&wb)[V_KC / 2]) {
  const int64_t c = (k0 / V_KC) * a.wld;
  const uint4* ps = reinterpret_cast<const uint4*>(ws + c);
  const uint4* pe = reinterpret_cast<const uint4*>(we + c);
#pragma unroll
  for (int i = 0; i < V_KC / 4; ++i) {
    const uint4 v = ps[i * 64];
    wa[4 * i] = v.x; wa[4 * i + 1] = v.y; wa[4 * i + 2] = v.z; wa[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < V_KC / 8; ++i) {
    const uint4 v = pe[i * 64];
    wb[4 * i] = v.x; wb[4 * i + 1] = v.y; wb[4 * i + 2] = v.z; wb[4 * i + 3] = v.w;
  }
}

// R rows (2) and 64 columns per workgroup of W waves; PRE: w comes
// pre-decoded from the workspace.  Epilogue EPI_STORE or EPI_ADD.
template <int DT, bool PRE, int R, bool PAIR, int W, int WPE>
__global__ __launch_bounds__(64 * W, WPE) void k_partial(GemmArgs a, const void* __restrict__ xg,
                                                         const void* __restrict__ wg) {
  constexpr int SLOT = R * 64 * (PAIR ? 8 : 4);   // bytes between slots
  __shared__ __align__(16) char cnt[NSLOT * SLOT];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t tile = xcd_tile();
  const int64_t m0 = (tile % a.tiles_m) * R, n0 = (tile / a.tiles_m) * V_BN;

  for (int q = threadIdx.x; q < NSLOT * SLOT / 16; q += 64 * W)
    reinterpret_cast<uint4*>(cnt)[q] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();

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
  const int xj = lane & 15;
  const uint32_t xj4 = static_cast<uint32_t>(xj) * 4u;
  const uint32_t lane_off = static_cast<uint32_t>(lane * (PAIR ? 8 : 4));
  const int32_t* const wsl = a.wsig + n0 * V_KC + lane * 4;     // the lane's sub-block 0 of chunk 0
  const uint16_t* const wel = a.wexp + n0 * V_KC + lane * 8;

  const int64_t nchunks = (a.K + V_KC - 1) / V_KC;
  uint32_t wq[2][V_KC], wbq[2][V_KC / 2], xq[2][R], xwq[2][R];
#pragma unroll
  for (int i = 0; i < V_KC / 2; ++i) { wbq[0][i] = 0u; wbq[1][i] = 0u; }
#pragma unroll
  for (int r = 0; r < R; ++r) xq[0][r] = xq[1][r] = xwq[0][r] = xwq[1][r] = 0u;
  constexpr int64_t ESZ = DT == DET_F32 ? 4 : 2;
  const char* const xp = static_cast<const char*>(xg) + (xrow[0] + xj * a.x_sk) * ESZ;
  const int64_t xstep = V_KC * a.x_sk * ESZ, xrstep = a.x_sm * ESZ;
  const bool rows_in = m0 + R <= a.M;
  auto load = [&](int64_t c, uint32_t (&w)[V_KC], uint32_t (&we)[V_KC / 2], uint32_t (&x)[R], uint32_t (&xw)[R]) {
    const int64_t k0 = c * V_KC;
    if (PRE) load_w_pre(a, wsl, wel, k0, w, we);
    else load_w_chunk<DT>(a, wg, wrow, n_ok, k0, w);
    if (PRE) {                                    // decoded x: padded, no masking
      const char* const xb = reinterpret_cast<const char*>(a.xsig + m0 * a.xld + k0);
      const char* const wb = reinterpret_cast<const char*>(a.xword + m0 * a.xld + k0);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        x[r] = *reinterpret_cast<const uint32_t*>(xb + r * a.xld * 4 + xj4);
        xw[r] = *reinterpret_cast<const uint32_t*>(wb + r * a.xld * 4 + xj4);
      }
    } else if (k0 + V_KC <= a.K && rows_in) {
      const char* const p = xp + c * xstep;
#pragma unroll
      for (int r = 0; r < R; ++r) x[r] = load_elem<DT>(p + r * xrstep, 0);
    } else {
      const int64_t k = min<int64_t>(k0 + xj, a.K - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) x[r] = load_elem<DT>(xg, xrow[r] + k * a.x_sk);
    }
  };
  if (wave < nchunks) load(wave, wq[0], wbq[0], xq[0], xwq[0]);

  // this wave's chunks: wave, wave + W, ...; in pairs so that the ring slot of
  // each is static
  for (int64_t c0 = wave; c0 < nchunks; c0 += 2 * W) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int64_t c = c0 + sl * W;
      if (c >= nchunks) break;
      if (c + W < nchunks) load(c + W, wq[sl ^ 1], wbq[sl ^ 1], xq[sl ^ 1], xwq[sl ^ 1]);
      const bool kin = c * V_KC + xj < a.K;
      int xm[R], xe[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        int32_t m;
        uint32_t e;
        if (PRE) { m = static_cast<int32_t>(xq[sl][r]); e = xwq[sl][r]; }
        else decode<DT, false, 0, EXP_SHIFT>(kin && row_ok[r] ? xq[sl][r] : 0u, m, e);
        xm[r] = m;
        xe[r] = static_cast<int>(e);
      }
      // f32, pre-decoded: x's significands by scalar loads (the chunk is the
      // same in every lane), SGPR operands of the products (no broadcast)
      constexpr bool SX = PRE && DT == DET_F32;
      uint32_t xs[R][V_KC];
      if constexpr (SX) {
        const int64_t cu = __builtin_amdgcn_readfirstlane(static_cast<int>(c));
        typedef const __attribute__((address_space(4))) uint32_t* cword;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const cword q = (cword)(a.xsig + (m0 + r) * a.xld + cu * V_KC);
#pragma unroll
          for (int i = 0; i < V_KC; ++i) xs[r][i] = q[i];
        }
      }
      steps_raw<DT, R, PRE, PAIR, SX, 0>(cnt, lane_off, wq[sl], wbq[sl], xm, xe, xs);
    }
  }
  __syncthreads();

  // wave r turns row r's counters into digits
  const int r = wave;
  if (r >= R || !n_ok || !(m0 + r < a.M)) return;
  const int64_t m = m0 + r;
  int64_t* const d = a.acc + (m * a.N + n) * ND;
  if constexpr (PAIR) {
    // field f = low half of slot f + high half of slot f - 1, positive minus
    // negative; digit j = field 2j + 2^16 field 2j+1
    const unsigned long long* const q = reinterpret_cast<const unsigned long long*>(cnt + lane * 8);
    constexpr int FQ = SLOT / 8;
    auto field = [&](int f) -> int64_t {
      if (f >= NF) return 0;
      const unsigned long long p0 = q[f * FQ], n0 = q[(NEG_SLOT + f) * FQ];
      int64_t v = static_cast<int64_t>(static_cast<uint32_t>(p0)) - static_cast<int64_t>(static_cast<uint32_t>(n0));
      if (f > 0) v += static_cast<int64_t>(q[(f - 1) * FQ] >> 32) - static_cast<int64_t>(q[(NEG_SLOT + f - 1) * FQ] >> 32);
      return v;
    };
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const int64_t v = field(2 * j) + field(2 * j + 1) * 65536;
      d[j] = a.epi == EPI_ADD ? d[j] + v : v;
    }
    return;
  }
  const int* const c = reinterpret_cast<const int*>(cnt + r * 256 + lane * 4);
  constexpr int F = SLOT / 4;
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    const int64_t lo = static_cast<int64_t>(c[(2 * j) * F]) - c[(NEG_SLOT + 2 * j) * F];
    const int64_t hi = 2 * j + 1 < NF ? static_cast<int64_t>(c[(2 * j + 1) * F]) - c[(NEG_SLOT + 2 * j + 1) * F] : 0;
    const int64_t v = lo + hi * 65536;
    d[j] = a.epi == EPI_ADD ? d[j] + v : v;
  }
}

// ---------------------------------------------------------------- det_gemm kernel
//
// det_gemm needs only the exact sum, not the raw digits, so a product may go
// into the accumulator in any pieces whose values add up to it.  Here it goes
// whole, with ONE LDS atomic, into one cell of a fixed grid: cell c of an
// output weighs 2^(B*c - 298) and takes T = P * 2^s, P the product of the
// (sign-applied) significands and s the product's bit offset o modulo B.
// Two grids (the traits below):
//   CellsG<f32, 2, 4> (f32, what det_gemm runs): B = 4, cell o div 4, s = o
//     mod 4 applied per product; |P| < 2^48, so |T| < 2^51 and the cells are
//     int64 (ds_add_u64), 4096 adds between folds, 128 cells (o <= 508).
//     Exponent words carry o * stride / 4, so the cell's byte offset is
//     o & ~(stride - 1) (one and-or with the lane's offset) and s one
//     bit-field extract.  (CellsG with B = 8 is the 8-bit form: 256 adds
//     between folds, 64 cells.)
//   Cells4 (bf16): B = 4, and each side's exponent is split into a cell part
//     and a 2-bit shift that is applied to that side's significand when it is
//     decoded: ex = 4cx + sx, ew = 4cw + sw, x' = x_sig << sx, w' = w_sig <<
//     sw, |x'|, |w'| < 2^11, so T = x' * w' has |T| < 2^22 and goes into cell
//     cx + cw.  Both sides also carry their part of the byte address (x: the
//     cell part and the row, w: the cell part and the lane), so one DPP add
//     gives the address and one 24-bit multiply the value: two VALU
//     instructions per product.  int32 cells, 512 adds between folds, 128
//     cells (offsets 32..538 are cells 7..134).
//
// The cells of R x 64 outputs fill R x 64 KB (f32) or R x 32 KB (bf16): too
// much for one wave if the CU is to hold enough waves to keep its VALUs busy,
// so W waves share them (f32: 2 rows, 128 KB, 16 waves, one workgroup per
// CU; bf16: 2 rows, 64 KB, 8 waves, two workgroups per CU).  A workgroup owns
// rows m0..m0+R-1 and 64 columns; its waves take the K-chunks in turn (wave
// v: chunks v, v + W, ...) and all add into the same cells, which the LDS
// atomics keep exact.  At the end of every epoch (the adds a cell can take)
// the workgroup meets at a barrier, each wave folds its 1/W of the cells into
// a window of int64 digits in its registers and clears them, and a second
// barrier opens the next epoch.  At the end the windows are added into one
// digit array per row in LDS and waves 0..R-1 finish the rows (round to fp32,
// or carry the digits to the next K block).

template <int DT, int R, int B>
struct CellsG {
  static_assert(B == 4 || B == 8, "cell grids of 4 or 8 bits");
  static constexpr int ROWS = R;
  static constexpr bool XPACK = false;          // decoded x: separate significand and word arrays
  static constexpr int NCELL = 512 / B;         // cells that products reach
  static constexpr int FIRST = DT == DET_F32 ? 0 : 32 / B;   // first reachable cell (bf16: offset >= 32)
  static constexpr int BITS = B;
  static constexpr int ES = DT == DET_F32 ? 8 : 4;        // bytes per cell
  static constexpr int RB = 64 * ES;                      // bytes between rows
  static constexpr uint32_t CS = R * RB;                  // bytes between cells
  static constexpr int ALLOC = FIRST + NCELL;             // cells allocated (the first FIRST unused)
  static constexpr int64_t KFLUSH = B == 8 ? 256 : 4096;  // adds between folds: |T| < 2^(47 + B)
  static constexpr int NORM_EVERY = B == 8 ? 8 : 1;       // folds between carry passes
  static constexpr bool CLAIM = true;                     // waves claim chunks (one workgroup per CU)
  // pre-decoded x significands through scalar loads: every lane multiplies
  // the same x element, so it is an SGPR operand of the multiply and needs no
  // broadcast (f32; bf16 packs significand and word in one word)
  static constexpr bool SX = DT == DET_F32;
  static constexpr uint32_t ESH = (DT == DET_F32 ? 9u : 8u) - (B == 8 ? 3u : 2u) +
                                  (R == 4 ? 2u : R == 2 ? 1u : 0u);   // log2(CS / B)
  static_assert(R == 1 || R == 2 || R == 4, "the cell stride must be a power of two");
  using cell_t = typename std::conditional<DT == DET_F32, int64_t, int32_t>::type;

  __device__ static void decode_x(uint32_t b, int /*r*/, int32_t& m, uint32_t& e) {
    decode<DT, true, 0, ESH>(b, m, e);
  }
  __device__ static void decode_w(uint32_t b, uint32_t /*lane*/, int32_t& m, uint32_t& e) {
    decode<DT, true, 1, ESH>(b, m, e);
  }
  // one product; xm, xe are x's (already broadcast) significand and word
  __device__ static void step(char* cbase, uint32_t lane_off, int r, int xm, uint32_t xe, int32_t wm,
                              uint32_t we) {
    const uint32_t o = xe + we;
    char* const p = cbase + ((o & ~(CS - 1u)) | (lane_off + r * RB));
    const uint32_t sh = (o >> ESH) & static_cast<uint32_t>(B - 1);
    if (DT == DET_F32) {
      const uint64_t T = static_cast<uint64_t>(static_cast<int64_t>(xm) * wm) << sh;
      atomicAdd(reinterpret_cast<unsigned long long*>(p), static_cast<unsigned long long>(T));
    } else {
      atomicAdd(reinterpret_cast<int*>(p), static_cast<int>(static_cast<uint32_t>(__mul24(xm, wm)) << sh));
    }
  }
};

template <int DT, int R>
using Cells8 = CellsG<DT, R, 8>;

template <int R>
struct Cells4 {
  static constexpr int ROWS = R;
  // decoded x packs the 12-bit shifted significand and the address word
  // (< 2^17) into one 32-bit word: one load per row and chunk, two
  // instructions to unpack
  static constexpr bool XPACK = true;
  __device__ static uint32_t pack_x(int32_t m, uint32_t e) { return (e << 12) | (static_cast<uint32_t>(m) & 0xFFFu); }
  __device__ static void unpack_x(uint32_t w, int32_t& m, uint32_t& e) {
    m = static_cast<int32_t>(w << 20) >> 20;
    e = w >> 12;
  }
  static constexpr int NCELL = 128;
  static constexpr int FIRST = 7;                         // offsets >= 32 -> cells >= 7
  static constexpr int BITS = 4;
  static constexpr int ES = 4;
  static constexpr int RB = 64 * ES;
  static constexpr uint32_t CS = R * RB;
  static constexpr int ALLOC = NCELL;                     // addresses are rebased to cell 7
  static constexpr int64_t KFLUSH = 512;
  static constexpr int NORM_EVERY = 1;
  static constexpr bool CLAIM = false;                    // fixed chunk shares (two workgroups per CU)
  static constexpr bool SX = false;
  using cell_t = int32_t;

  // bf16 bits -> shifted significand and address word.  x: exponent offset
  // ex = max(E,1) + 30 (31..284), word (ex div 4 - 7) * CS + row offset;
  // w: ew = max(E,1) (1..254), word ew div 4 * CS + lane offset.  The two
  // words add up to (o div 4 - 7) * CS + row + lane, o = ex + ew, within the
  // 128 cells.
  __device__ static void decode_x(uint32_t b, int r, int32_t& m, uint32_t& e) {
    const uint32_t E = (b >> 7) & 0xFFu;
    const uint32_t mag = (b & 0x7Fu) | (min(E, 1u) << 7);
    const uint32_t ex = max(E, 1u) + 30u;
    const uint32_t neg = (b >> 15) & 1u, sgn = 0u - neg;
    m = static_cast<int32_t>(((mag << (ex & 3u)) ^ sgn) + neg);
    e = ((ex >> 2) - FIRST) * CS + static_cast<uint32_t>(r) * RB;
  }
  __device__ static void decode_w(uint32_t b, uint32_t lane, int32_t& m, uint32_t& e) {
    const uint32_t E = (b >> 7) & 0xFFu;
    const uint32_t mag = (b & 0x7Fu) | (min(E, 1u) << 7);
    const uint32_t ew = max(E, 1u);
    const uint32_t neg = (b >> 15) & 1u, sgn = 0u - neg;
    m = static_cast<int32_t>(((mag << (ew & 3u)) ^ sgn) + neg);
    e = (ew >> 2) * CS + lane * 4u;
  }
  __device__ static void step(char* cbase, uint32_t /*lane_off*/, int /*r*/, int xm, uint32_t xe, int32_t wm,
                              uint32_t we) {
    atomicAdd(reinterpret_cast<int*>(cbase + (xe + we)), __mul24(xm, wm));
  }
};

template <class G>
__device__ __forceinline__ void unpack_packed(uint32_t w, int32_t& m, uint32_t& e) {
  if constexpr (G::XPACK) G::unpack_x(w, m, e);
}

// the lane's pre-decoded w chunk for k_gemm8: 16 significands and 16 32-bit
// words, both laid out like load_w_pre's 32-bit words
__device__ __forceinline__ void load_w_pre8(const GemmArgs& a, const int32_t* ws, const uint32_t* we, int64_t k0,
                                            uint32_t (&wa)[V_KC], uint32_t (&wb)[V_KC]) {
  const int64_t c = (k0 / V_KC) * a.wld;
  const uint4* ps = reinterpret_cast<const uint4*>(ws + c);
  const uint4* pe = reinterpret_cast<const uint4*>(we + c);
#pragma unroll
  for (int i = 0; i < V_KC / 4; ++i) {
    const uint4 v = ps[i * 64], e = pe[i * 64];
    wa[4 * i] = v.x; wa[4 * i + 1] = v.y; wa[4 * i + 2] = v.z; wa[4 * i + 3] = v.w;
    wb[4 * i] = e.x; wb[4 * i + 1] = e.y; wb[4 * i + 2] = e.z; wb[4 * i + 3] = e.w;
  }
}

// The workgroup's chunk counter, through a register that the compiler cannot
// see is the same in every lane.  lane 0's add on it then stays a single
// ds_add_rtn_u32; on a visibly uniform address the compiler wraps the add in
// a wave-wide count of the active lanes (about six vector instructions).
__device__ __forceinline__ int* claim_counter(int& claim) {
  uint32_t z = 0;
  asm volatile("" : "+v"(z));
  return &claim + z;
}

// lane 0 takes the next chunk from the counter; the other lanes get 0
__device__ __forceinline__ int claim_chunk(int* counter, uint32_t lane) {
  int got = 0;
  if (lane == 0) got = atomicAdd(counter, 1);
  return got;
}

// One chunk: step J takes x element J of each row (DPP broadcast from lane J
// of every 16-lane row) and the lane's w element J.
template <class G, int DT, bool PRE, int R, int J>
__device__ __forceinline__ void steps8(char* cbase, uint32_t lane, uint32_t lane_off, const uint32_t (&wa)[V_KC],
                                       const uint32_t (&wb)[V_KC], const int (&xm)[R], const int (&xe)[R],
                                       const uint32_t (&xs)[R][V_KC]) {
  int32_t wm;
  uint32_t we;
  if (PRE) {
    wm = static_cast<int32_t>(wa[J]);
    we = wb[J];
  } else {
    G::decode_w(wa[J], lane, wm, we);
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    G::step(cbase, lane_off, r, PRE && G::SX ? static_cast<int>(xs[r][J]) : bcast<J>(xm[r]),
            static_cast<uint32_t>(bcast<J>(xe[r])), wm, we);
  if constexpr (J + 1 < V_KC) steps8<G, DT, PRE, R, J + 1>(cbase, lane, lane_off, wa, wb, xm, xe, xs);
}

// dg += v * scale for a 32-bit v (unsigned or signed) and a power-of-two
// scale.  The compiler turns a multiply by a known power of two into a
// widen, a 64-bit shift and an add; hiding only the scale's value (an empty
// asm statement that emits no instruction) leaves it one v_mad_u64_u32 /
// v_mad_i64_i32 per call.  Every instruction is the compiler's own, so its
// hazard recognizer sees all of them: an earlier form issued these two mads
// from inline assembly, whose VALU writes (64-bit VGPRs and an SGPR carry
// pair) the recognizer cannot see.
__device__ __forceinline__ uint32_t opaque_scale(uint32_t scale) {
  asm("" : "+s"(scale));
  return scale;
}
__device__ __forceinline__ void mad_u32(int64_t& dg, uint32_t v, uint32_t scale) {
  dg = static_cast<int64_t>(static_cast<uint64_t>(dg) + static_cast<uint64_t>(v) * opaque_scale(scale));
}
__device__ __forceinline__ void mad_i32(int64_t& dg, int32_t v, uint32_t scale) {
  dg += static_cast<int64_t>(v) * static_cast<int32_t>(opaque_scale(scale));
}

// Fold the CW cells this wave owns (CW consecutive cells of this lane and
// row, starting at `c0`) into its window and clear them.  Window digit 0
// weighs 2^(32 jb) with jb = (first cell's bit position) div 32; cell i of
// the wave sits OFF + B*i bits above it, OFF the same for every wave.  With
// `norm`, carry the window so that all but its top digit lie in [0, 2^32).
template <class G, int CW, int OFF, int WD>
__device__ __forceinline__ void fold8(char* c0, int64_t (&dg)[WD], bool norm) {
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    const int bit = OFF + G::BITS * i;
    const uint32_t scale = 1u << (bit & 31);
    if (sizeof(typename G::cell_t) == 8) {
      int64_t* q = reinterpret_cast<int64_t*>(c0 + i * G::CS);
      const int64_t v = *q;
      *q = 0;
      mad_u32(dg[bit >> 5], static_cast<uint32_t>(v), scale);
      mad_i32(dg[(bit >> 5) + 1], static_cast<int32_t>(v >> 32), scale);
    } else {
      int* q = reinterpret_cast<int*>(c0 + i * G::CS);
      mad_i32(dg[bit >> 5], *q, scale);
      *q = 0;
    }
    // keep the scheduler from reading many cells ahead (register pressure)
    if ((i & 3) == 3) asm volatile("" ::: "memory");
  }
  if (norm) {
#pragma unroll
    for (int j = 0; j + 1 < WD; ++j) {
      const int64_t carry = dg[j] >> 32;
      dg[j] -= carry * (int64_t(1) << 32);
      dg[j + 1] += carry;
    }
  }
}

// One R x 64 output tile of det_gemm: the body of k_gemm8.
template <class G, int DT, bool PRE, int R, int W>
__device__ __forceinline__ void gemm8_tile(const GemmArgs& a, const void* __restrict__ xg,
                                           const void* __restrict__ wg, int64_t tile, int tid, bool fresh, char* cells,
                                           int& claim) {
  constexpr int CW = G::NCELL / W;                          // cells each wave folds
  constexpr int OFF = (G::BITS * G::FIRST) & 31;            // bit of a wave's first cell within its digit
  // window digits: the window's value stays below 2^(OFF + B(CW-1) + cell
  // bits + log2 CW + 1), so this many digits hold it with the top one signed
  constexpr int VB = sizeof(typename G::cell_t) == 8 ? 63 : 31;
  constexpr int LOG2CW = CW <= 1 ? 0 : CW <= 2 ? 1 : CW <= 4 ? 2 : CW <= 8 ? 3 : CW <= 16 ? 4 : 5;
  constexpr int WD = (OFF + G::BITS * (CW - 1) + VB + LOG2CW + 1 + 31) / 32;
  constexpr int64_t EPOCH = G::KFLUSH / V_KC;               // chunks per epoch, all waves together
  static_assert(CW * W == G::NCELL && EPOCH >= W && (G::BITS * CW) % 32 == 0, "epoch layout");

  const int lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = (tile % a.tiles_m) * R, n0 = (tile / a.tiles_m) * V_BN;


  const int64_t n = n0 + lane;
  const bool n_ok = n < a.N;
  // raw operands: rows and columns through the maps (pre-decoded ones were
  // gathered by the decode)
  const int64_t wn = n_ok ? n : a.N - 1;
  const int64_t wrow = (!PRE && a.wmap != nullptr ? a.wmap[wn] : wn) * a.w_sn;
  bool row_ok[R];
  int64_t xrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    row_ok[r] = m0 + r < a.M;
    const int64_t mr = min(m0 + r, a.M - 1);
    xrow[r] = (!PRE && a.xmap != nullptr ? a.xmap[mr] : mr) * a.x_sm;
  }
  const int xj = lane & 15;
  const uint32_t xj4 = static_cast<uint32_t>(xj) * 4u;
  const uint32_t lane_off = static_cast<uint32_t>(lane * G::ES);


  const int64_t nchunks = (a.K + V_KC - 1) / V_KC;
  uint32_t wq[2][V_KC], weq[2][V_KC], xq[2][R], xwq[2][R];
#pragma unroll
  for (int i = 0; i < V_KC; ++i) { weq[0][i] = 0u; weq[1][i] = 0u; }
#pragma unroll
  for (int r = 0; r < R; ++r) xq[0][r] = xq[1][r] = xwq[0][r] = xwq[1][r] = 0u;
  // x element k0 + xj of each row: a per-lane pointer plus a wave-uniform
  // chunk offset, clamped into the row only in the last, partial chunk
  constexpr int64_t ESZ = DT == DET_F32 ? 4 : 2;
  const char* const xp = static_cast<const char*>(xg) + (xrow[0] + xj * a.x_sk) * ESZ;
  const int64_t xstep = V_KC * a.x_sk * ESZ, xrstep = a.x_sm * ESZ;
  const bool rows_in = m0 + R <= a.M && (PRE || a.xmap == nullptr);   // all R rows exist, x_sm apart
  const int32_t* const wsl = a.wsig + n0 * V_KC + lane * 4;       // the lane's sub-block 0 of chunk 0
  const uint32_t* const wel = a.wexp32 + n0 * V_KC + lane * 4;
  auto load = [&](int64_t c, uint32_t (&w)[V_KC], uint32_t (&we)[V_KC], uint32_t (&x)[R], uint32_t (&xw)[R]) {
    const int64_t k0 = c * V_KC;
    if (PRE) load_w_pre8(a, wsl, wel, k0, w, we);
    else load_w_chunk<DT>(a, wg, wrow, n_ok, k0, w);
    if (PRE) {                                    // decoded x: padded, no masking
      const char* const xb = reinterpret_cast<const char*>(a.xsig + m0 * a.xld + k0);
      const char* const wb = reinterpret_cast<const char*>(a.xword + m0 * a.xld + k0);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (!G::SX) x[r] = *reinterpret_cast<const uint32_t*>(xb + r * a.xld * 4 + xj4);
        if (!G::XPACK) xw[r] = *reinterpret_cast<const uint32_t*>(wb + r * a.xld * 4 + xj4);
      }
    } else if (k0 + V_KC <= a.K && rows_in) {
      const char* const p = xp + c * xstep;
#pragma unroll
      for (int r = 0; r < R; ++r) x[r] = load_elem<DT>(p + r * xrstep, 0);
    } else {
      const int64_t k = min<int64_t>(k0 + xj, a.K - 1);
#pragma unroll
      for (int r = 0; r < R; ++r) x[r] = load_elem<DT>(xg, xrow[r] + k * a.x_sk);
    }
  };
  // the first chunk's loads go out before the cells are cleared.  After a
  // tile of this workgroup (`fresh` false) the folds have zeroed every cell,
  // and only the digit array laid over the first cells needs clearing.
  if (wave < nchunks) load(wave, wq[0], weq[0], xq[0], xwq[0]);
  const int clear16 = fresh ? G::ALLOC * static_cast<int>(G::CS) / 16 : R * ND * 64 * 8 / 16;
  for (int q = tid; q < clear16; q += 64 * W)
    reinterpret_cast<uint4*>(cells)[q] = make_uint4(0u, 0u, 0u, 0u);
  if (tid == 0) claim = W;
  __syncthreads();

  // this wave's cells: CW consecutive cells from cell FIRST + wave * CW
  char* const my_cells = cells + (G::ALLOC - G::NCELL + wave * CW) * G::CS + lane * G::ES;
  // Epochs of EPOCH chunks.  The barriers stay outside the unrolled pairs of
  // ring slots, so every wave meets each of them once per epoch.
  // One chunk of products from ring slot sl.
  // chunk c from ring slot sl
  auto compute = [&](int64_t c, int sl) {
    const bool kin = c * V_KC + xj < a.K;
    int xm[R], xe[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int32_t m;
      uint32_t e;
      if (PRE && G::XPACK) unpack_packed<G>(xq[sl][r], m, e);
      else if (PRE) { m = static_cast<int32_t>(xq[sl][r]); e = xwq[sl][r]; }
      else G::decode_x(kin && row_ok[r] ? xq[sl][r] : 0u, r, m, e);
      xm[r] = m;
      xe[r] = static_cast<int>(e);
    }
    uint32_t xs[R][V_KC];
    if constexpr (PRE && G::SX) {
      // the chunk's x significands by scalar loads (the chunk index is the
      // same in every lane), just before its products
      const int64_t cu = __builtin_amdgcn_readfirstlane(static_cast<int>(c));
      typedef const __attribute__((address_space(4))) uint32_t* cword;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const cword q = (cword)(a.xsig + (m0 + r) * a.xld + cu * V_KC);
#pragma unroll
        for (int i = 0; i < V_KC; ++i) xs[r][i] = q[i];
      }
    }
    steps8<G, DT, PRE, R, 0>(cells, static_cast<uint32_t>(lane), lane_off, wq[sl], weq[sl], xm, xe, xs);
  };
  // An epoch's chunks e0 .. e0 + lim - 1: wave v starts with chunk e0 + v
  // (already in ring slot 0).  With G::CLAIM it then takes the next unclaimed
  // one from the counter `claim`: the CU serves its waves unequally (older
  // first), so with one workgroup per CU a fixed share per wave leaves the
  // early ones idle at the barrier while the late ones finish, and claiming
  // keeps them all busy to the end (f32: 17.0 -> 16.2 ms on 4096^3).  Each
  // claim is made one chunk ahead: its result is read a whole chunk of
  // products later.  Without it (bf16: two workgroups per CU fill each
  // other's tails, and the claim cost 6 % there) wave v takes chunks e0 + v +
  // i*W.
  auto run_epoch = [&](int64_t e0) {
    const int lim = static_cast<int>(min<int64_t>(nchunks - e0, EPOCH));
    int cur = wave;
    if (cur >= lim) return;
    if constexpr (!G::CLAIM) {
      // fixed shares: wave v takes chunks e0 + v + i*W; the two ring slots
      // written out (constant slot indices keep the ring in registers)
      auto slot = [&](auto slc) {
        constexpr int sl = decltype(slc)::value;
        const int nxt = cur + W;
        if (nxt < lim) load(e0 + nxt, wq[sl ^ 1], weq[sl ^ 1], xq[sl ^ 1], xwq[sl ^ 1]);
        compute(e0 + cur, sl);
        cur = nxt;
        return nxt >= lim;
      };
#pragma unroll 1
      for (;;) {
        if (slot(std::integral_constant<int, 0>{})) return;
        if (slot(std::integral_constant<int, 1>{})) return;
      }
    }
    int* const counter = claim_counter(claim);
    // lane 0's claim, as a scalar: the chunk's addresses are then scalar
    // arithmetic, where a shuffle would leave them to per-lane 64-bit VALU work
    int nxt = __builtin_amdgcn_readfirstlane(claim_chunk(counter, static_cast<uint32_t>(lane)));
#pragma unroll 1
    for (;;) {
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const int pend = nxt < lim ? claim_chunk(counter, static_cast<uint32_t>(lane)) : 0;
        if (nxt < lim) load(e0 + nxt, wq[sl ^ 1], weq[sl ^ 1], xq[sl ^ 1], xwq[sl ^ 1]);
        compute(e0 + cur, sl);
        if (nxt >= lim) return;
        cur = nxt;
        nxt = __builtin_amdgcn_readfirstlane(pend);
      }
    }
  };
  // The first epoch is peeled off: its fold defines the windows, so they
  // hold no registers during its adds (with 16 waves per CU they would spill,
  // and a 4096-long K is a single epoch on the 4-bit grid).
  run_epoch(0);
  __syncthreads();                                // the epoch's adds are in
  if (tid == 0) claim = W;
  if (EPOCH + wave < nchunks) load(EPOCH + wave, wq[0], weq[0], xq[0], xwq[0]);
  int64_t dg[R][WD];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int j = 0; j < WD; ++j) dg[r][j] = 0;
    fold8<G, CW, OFF, WD>(my_cells + r * G::RB, dg[r], G::NORM_EVERY == 1 || EPOCH >= nchunks);
  }
  __syncthreads();                                // cells clear before the next epoch
  int64_t epoch = 1;
  for (int64_t e0 = EPOCH; e0 < nchunks; e0 += EPOCH, ++epoch) {
    run_epoch(e0);
    __syncthreads();                              // the epoch's adds are in
    if (tid == 0) claim = W;
    if (e0 + EPOCH + wave < nchunks) load(e0 + EPOCH + wave, wq[0], weq[0], xq[0], xwq[0]);
    const bool norm = (epoch % G::NORM_EVERY) == G::NORM_EVERY - 1 || e0 + EPOCH >= nchunks;
#pragma unroll
    for (int r = 0; r < R; ++r) fold8<G, CW, OFF, WD>(my_cells + r * G::RB, dg[r], norm);
    __syncthreads();                              // cells clear before the next epoch
  }

  // windows -> one digit array per row in LDS (over the cells, all zero now)
  int64_t* const D = reinterpret_cast<int64_t*>(cells);        // D[(r * ND + j) * 64 + lane]
  static_assert(R * ND * 64 * 8 <= G::ALLOC * G::CS, "digit array fits over the cells");
  const int jb = (G::BITS * (G::FIRST + wave * CW)) >> 5;      // window digit 0 in the accumulator
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int d = WD - 1; d > 0; --d)              // anything beyond digit ND-1 joins digit ND-1
      if (jb + d >= ND) { dg[r][d - 1] += dg[r][d] * (int64_t(1) << 32); dg[r][d] = 0; }
#pragma unroll
    for (int d = 0; d < WD; ++d)
      if (jb + d < ND) atomicAdd(reinterpret_cast<unsigned long long*>(D + (r * ND + jb + d) * 64 + lane),
                                 static_cast<unsigned long long>(dg[r][d]));
  }
  __syncthreads();
  // wave r finishes row r
  const int r = wave;
  if (r >= R || !n_ok || !(m0 + r < a.M)) return;
  const int64_t m = m0 + r;
  int64_t acc[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) acc[j] = D[(r * ND + j) * 64 + lane];
  int64_t* dd = a.acc + (m * a.N + n) * ND;
  if (a.epi == EPI_ADD || a.epi == EPI_ADD_ROUND) {
#pragma unroll
    for (int j = 0; j < ND; ++j) acc[j] += dd[j];
  }
  if (a.epi == EPI_STORE || a.epi == EPI_ADD) {
#pragma unroll
    for (int j = 0; j < ND; ++j) dd[j] = acc[j];
  } else {
    const int64_t ym = a.xmap != nullptr ? a.xmap[m] : m, yn = a.wmap != nullptr ? a.wmap[n] : n;
    a.y[ym * a.y_sm + yn * a.y_sn] = __uint_as_float(round_digits_to_f32(acc));
  }
}

// The pre-decoded f32 form of k_gemm8 (one workgroup per CU, waves
// claiming chunks) over a workgroup's consecutive tiles t0 .. t1-1, with
// two barriers per tile: after the epoch's adds, and after the digit sums.
// Between them every wave issues the loads of the next tile's first chunk
// (so they are in flight while it folds), folds its cells into its windows
// (leaving the cells zero) and adds the windows into the digit array D, which
// has its own LDS beside the cells.  After the second barrier waves 0 .. R-1
// read their rows of D, clear them and round, while the other waves already
// add the next tile's products; the claims let the late waves take fewer
// chunks.  Nothing waits for the rounding and its y store, and no tile but
// the first clears LDS.
template <class G, int DT, int R, int W>
__device__ __forceinline__ void gemm8_claim_tiles(const GemmArgs& a, int t0, int t1, char* cells, int64_t* D,
                                                  int& claim) {
  static_assert(G::CLAIM && G::SX && !G::XPACK, "the claiming form with x significands in SGPRs");
  constexpr int CW = G::NCELL / W;                          // cells each wave folds
  constexpr int OFF = (G::BITS * G::FIRST) & 31;            // bit of a wave's first cell within its digit
  constexpr int VB = sizeof(typename G::cell_t) == 8 ? 63 : 31;
  constexpr int LOG2CW = CW <= 1 ? 0 : CW <= 2 ? 1 : CW <= 4 ? 2 : CW <= 8 ? 3 : CW <= 16 ? 4 : 5;
  constexpr int WD = (OFF + G::BITS * (CW - 1) + VB + LOG2CW + 1 + 31) / 32;
  constexpr int64_t EPOCH = G::KFLUSH / V_KC;               // chunks per epoch, all waves together
  static_assert(CW * W == G::NCELL && EPOCH >= W && (G::BITS * CW) % 32 == 0, "epoch layout");

  // 32-bit tile, row, column and chunk indices (fewer SGPRs; tiles < 2^31,
  // K < 2^19 in one launch)
  const int nchunks = static_cast<int>((a.K + V_KC - 1) / V_KC);
  const int tm = static_cast<int>(a.tiles_m);
  // the thread's indices, re-derived at each tile (the lane from the exec
  // mask, the wave index from an SGPR opaque to the compiler): nothing
  // derived from them is hoisted out of the tile loop to hold registers, and
  // the thread index itself is not kept
  int wave0 = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  int tid, lane, wave;
  uint32_t xj4, lane_off;
  char* my_cells;
  int* counter;
  auto derive = [&]() {
    asm volatile("" : "+s"(wave0));
    wave = wave0;
    uint32_t ones = ~0u;
    asm volatile("" : "+s"(ones));
    lane = static_cast<int>(__builtin_amdgcn_mbcnt_hi(ones, __builtin_amdgcn_mbcnt_lo(ones, 0u)));
    tid = wave * 64 + lane;
    xj4 = static_cast<uint32_t>(lane & 15) * 4u;
    lane_off = static_cast<uint32_t>(lane * G::ES);
    my_cells = cells + (G::ALLOC - G::NCELL + wave * CW) * G::CS + lane * G::ES;
    counter = claim_counter(claim);
  };

  uint32_t wq[2][V_KC], weq[2][V_KC], xwq[2][R];
  const int xm0[R] = {};                          // unused: the significands come as SGPR operands

  // chunk c of the tile at (m0, n0): the lane's w chunk and x's words
  auto load = [&](int m0, int n0, int c, uint32_t (&w)[V_KC], uint32_t (&we)[V_KC], uint32_t (&xw)[R]) {
    const int64_t k0 = static_cast<int64_t>(c) * V_KC;
    load_w_pre8(a, a.wsig + static_cast<int64_t>(n0) * V_KC + lane * 4,
                a.wexp32 + static_cast<int64_t>(n0) * V_KC + lane * 4, k0, w, we);
    const char* const wb = reinterpret_cast<const char*>(a.xword + m0 * a.xld + k0);
#pragma unroll
    for (int r = 0; r < R; ++r) xw[r] = *reinterpret_cast<const uint32_t*>(wb + r * a.xld * 4 + xj4);
  };
  // chunk c from ring slot sl; the x significands by scalar loads (the chunk
  // index is the same in every lane), just before its products
  auto compute = [&](int m0, int c, int sl) {
    int xe[R];
#pragma unroll
    for (int r = 0; r < R; ++r) xe[r] = static_cast<int>(xwq[sl][r]);
    uint32_t xs[R][V_KC];
    const int64_t cu = __builtin_amdgcn_readfirstlane(c);
    typedef const __attribute__((address_space(4))) uint32_t* cword;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const cword q = (cword)(a.xsig + (m0 + r) * a.xld + cu * V_KC);
#pragma unroll
      for (int i = 0; i < V_KC; ++i) xs[r][i] = q[i];
    }
    steps8<G, DT, true, R, 0>(cells, static_cast<uint32_t>(lane), lane_off, wq[sl], weq[sl], xm0, xe, xs);
  };
  // an epoch's chunks e0 .. e0 + lim - 1: wave v starts with chunk e0 + v
  // (in ring slot 0), then takes the next unclaimed one, claimed a chunk ahead
  auto run_epoch = [&](int m0, int n0, int e0) {
    const int lim = min(nchunks - e0, static_cast<int>(EPOCH));
    int cur = wave;
    if (cur >= lim) return;
    // lane 0's claim, as a scalar: the chunk's addresses are then scalar
    // arithmetic, where a shuffle would leave them to per-lane 64-bit VALU work
    int nxt = __builtin_amdgcn_readfirstlane(claim_chunk(counter, static_cast<uint32_t>(lane)));
    // (the last chunk's products are written out apart, so that the other
    // slot is read only on the path that loaded it: the compiler then keeps
    // no ring slot but slot 0 live across tiles)
    auto slot = [&](auto slc) {
      constexpr int sl = decltype(slc)::value;
      if (nxt >= lim) {
        compute(m0, e0 + cur, sl);
        return true;
      }
      const int pend = claim_chunk(counter, static_cast<uint32_t>(lane));
      load(m0, n0, e0 + nxt, wq[sl ^ 1], weq[sl ^ 1], xwq[sl ^ 1]);
      compute(m0, e0 + cur, sl);
      cur = nxt;
      nxt = __builtin_amdgcn_readfirstlane(pend);
      return false;
    };
#pragma unroll 1
    for (;;) {
      if (slot(std::integral_constant<int, 0>{})) return;
      if (slot(std::integral_constant<int, 1>{})) return;
    }
  };

  // the tile's first row and column, stepped down the rows (column-major
  // tile order)
  int m0 = (t0 % tm) * R, n0 = (t0 / tm) * V_BN;
  for (int t = t0; t < t1; ++t) {
    derive();
    if (t == t0) {
      // the first tile: every cell and D clear, its first chunks in flight
      load(m0, n0, min(wave, nchunks - 1), wq[0], weq[0], xwq[0]);
      for (int q = tid; q < G::ALLOC * static_cast<int>(G::CS) / 16; q += 64 * W)
        reinterpret_cast<uint4*>(cells)[q] = make_uint4(0u, 0u, 0u, 0u);
      for (int q = tid; q < R * ND * 64 * 8 / 16; q += 64 * W)
        reinterpret_cast<uint4*>(D)[q] = make_uint4(0u, 0u, 0u, 0u);
      if (tid == 0) claim = W;
      __syncthreads();
    }
    const int jb = (G::BITS * (G::FIRST + wave * CW)) >> 5;    // window digit 0 in the accumulator
    // the next tile (after the last one: this one again, a wasted load)
    int m1 = m0, n1 = n0;
    if (t + 1 < t1) {
      m1 += R;
      if (m1 >= tm * R) { m1 = 0; n1 += V_BN; }
    }
    // Ring slot 0 is loaded on every path (chunk indices clamped into the
    // operands; a wave past the chunks never computes it), so no earlier
    // value of it stays live across the rounding.
    const int cw = min(wave, nchunks - 1);
    // after an epoch's adds: the claims restart, and the first chunks of the
    // next epoch, else (waves R..W-1) of the next tile, go out
    auto after_epoch = [&](int e1) {
      __syncthreads();                            // the epoch's adds are in
      if (tid == 0) claim = W;
      if (e1 < nchunks) load(m0, n0, min(e1 + wave, nchunks - 1), wq[0], weq[0], xwq[0]);
      else if (wave >= R) load(m1, n1, cw, wq[0], weq[0], xwq[0]);
    };
    // the first epoch is peeled off: its fold defines the windows, which
    // then hold no registers during its adds
    run_epoch(m0, n0, 0);
    after_epoch(EPOCH);
    int64_t dg[R][WD];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int j = 0; j < WD; ++j) dg[r][j] = 0;
      fold8<G, CW, OFF, WD>(my_cells + r * G::RB, dg[r], G::NORM_EVERY == 1 || EPOCH >= nchunks);
    }
    int epoch = 1;
    for (int e0 = static_cast<int>(EPOCH); e0 < nchunks; e0 += static_cast<int>(EPOCH), ++epoch) {
      __syncthreads();                            // cells clear before the epoch
      run_epoch(m0, n0, e0);
      after_epoch(e0 + EPOCH);
      const bool norm = (epoch % G::NORM_EVERY) == G::NORM_EVERY - 1 || e0 + EPOCH >= nchunks;
#pragma unroll
      for (int r = 0; r < R; ++r) fold8<G, CW, OFF, WD>(my_cells + r * G::RB, dg[r], norm);
    }
    // windows -> the rows' digit arrays D[(r * ND + j) * 64 + lane] (clear:
    // their readers cleared them before this tile's first barrier)
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int d = WD - 1; d > 0; --d)            // anything beyond digit ND-1 joins digit ND-1
        if (jb + d >= ND) { dg[r][d - 1] += dg[r][d] * (int64_t(1) << 32); dg[r][d] = 0; }
#pragma unroll
      for (int d = 0; d < WD; ++d)
        if (jb + d < ND) atomicAdd(reinterpret_cast<unsigned long long*>(D + (r * ND + jb + d) * 64 + lane),
                                   static_cast<unsigned long long>(dg[r][d]));
    }
    __syncthreads();                              // the digit sums are in, every cell is zero
    // wave r finishes row r and clears its part of D.  The digits stream
    // through the carry pass one at a time (32-bit words kept, not 64-bit
    // digits), with the workspace's digits added or stored on the way.
    if (wave < R) {
      const int r = wave;
      const int64_t m = m0 + r, n = n0 + lane;
      const bool ok = m < a.M && n < a.N;
      const bool add = ok && (a.epi == EPI_ADD || a.epi == EPI_ADD_ROUND);
      const bool store = ok && (a.epi == EPI_STORE || a.epi == EPI_ADD);
      int64_t* const dd = a.acc + (m * a.N + n) * ND;
      uint32_t wv[ND];
      int64_t carry = 0;
#pragma unroll
      for (int j = 0; j < ND; ++j) {
        int64_t v = D[(r * ND + j) * 64 + lane];
        D[(r * ND + j) * 64 + lane] = 0;
        if (add) v += dd[j];
        if (store) dd[j] = v;
        const int64_t u = v + carry;
        wv[j] = static_cast<uint32_t>(u);
        carry = u >> 32;                          // arithmetic: floor(u / 2^32)
      }
      if (ok && !(a.epi == EPI_STORE || a.epi == EPI_ADD)) {
        const int64_t ym = a.xmap != nullptr ? a.xmap[m] : m, yn = a.wmap != nullptr ? a.wmap[n] : n;
        a.y[ym * a.y_sm + yn * a.y_sn] = __uint_as_float(round_words_to_f32(wv, carry));
      }
      load(m1, n1, cw, wq[0], weq[0], xwq[0]);  // then the next tile's first chunk
    }
    m0 = m1;
    n0 = n1;
  }
}

// det_gemm: one workgroup per tile in the XCD-aware order.  LOOP: each
// workgroup takes tpw consecutive tiles of that order, with M and N from the
// device counts if given: every pre-decoded launch of the claiming (f32)
// kernel (gemm8_claim_tiles), and the launches whose work the device decides
// (a gated one, whose skipped workgroups then cost a tpw-th of a full grid's
// dispatch, and the recompute of device-counted rows or columns).  In
// gemm8_tile's loop a barrier sits between tiles: waves 0 and 1 read the
// digit array over the cells while the others would clear them.
template <class G, int DT, bool PRE, int R, int W, int WPE, bool LOOP>
__global__ __launch_bounds__(64 * W, WPE) void k_gemm8(GemmArgs a, const void* __restrict__ xg,
                                                       const void* __restrict__ wg) {
  __shared__ __align__(16) char cells[G::ALLOC * G::CS];
  __shared__ int claim;                           // the epoch's next unclaimed chunk (from e0)
  // the claiming form's digit array (beside the cells; one int64 elsewhere)
  __shared__ __align__(16) int64_t dsum[G::CLAIM && PRE ? R * ND * 64 : 1];
  if (a.gate != nullptr && *a.gate == 0) return;
  if constexpr (G::CLAIM && PRE) {
    int64_t t0 = xcd_tile(), t1 = t0 + 1;
    if constexpr (LOOP) {
      if (a.mcount != nullptr) a.M = *a.mcount;
      if (a.ncount != nullptr) a.N = *a.ncount;
      a.tiles_m = (a.M + R - 1) / R;
      a.tiles_n = (a.N + V_BN - 1) / V_BN;
      t0 *= a.tpw;
      t1 = min(t0 + a.tpw, a.tiles_m * a.tiles_n);
    }
    if (t0 < t1) gemm8_claim_tiles<G, DT, R, W>(a, static_cast<int>(t0), static_cast<int>(t1), cells, dsum, claim);
  } else if constexpr (!LOOP) {
    gemm8_tile<G, DT, PRE, R, W>(a, xg, wg, xcd_tile(), threadIdx.x, true, cells, claim);
  } else {
    if (a.mcount != nullptr) a.M = *a.mcount;
    if (a.ncount != nullptr) a.N = *a.ncount;
    a.tiles_m = (a.M + R - 1) / R;
    a.tiles_n = (a.N + V_BN - 1) / V_BN;
    const int64_t tiles = a.tiles_m * a.tiles_n;
    const int64_t t0 = xcd_tile() * a.tpw, t1 = min(t0 + a.tpw, tiles);
    for (int64_t t = t0; t < t1; ++t) {
      // the thread index, opaque to the compiler at each tile: nothing
      // derived from it is hoisted out of the loop to hold registers
      int tid = static_cast<int>(threadIdx.x);
      asm volatile("" : "+v"(tid));
      gemm8_tile<G, DT, PRE, R, W>(a, xg, wg, t, tid, t == t0, cells, claim);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------- w pre-decode
// w [N][K] (any strides) -> significands int32 and exponent words (uint16
// for k_gemm, uint32 for k_gemm8), +0 outside N x K.  Layout: chunk-major
// (the 16 k of one chunk for all rows, then the next chunk), each chunk by
// 64-column tile, each tile in 16-byte sub-blocks: [Kp/16][Np/64][4][64][4]
// for 32-bit words, [Kp/16][Np/64][2][64][8] for 16-bit ones.  A GEMM wave
// then reads w with 16-byte loads that each cover one contiguous 1 KiB, and
// spends no instructions on decoding it.
// (Row-major [Np][Kp] put each lane of a wave in its own 2 MiB page once K
// reached 2^19, and the GEMM ran at half speed.)
struct PredecodeArgs {
  const void* w; int64_t w_sn, w_sk;
  int64_t N, K, Np, Kp;
  int32_t* wsig; void* wexp;          // exponent words: uint16 (k_gemm) or uint32 (k_gemm8)
  const int32_t* rmap;                // k_predecode_w8: decoded row n is row rmap[n] of w (null: n)
  // k_predecode_w8 decided on the device (null: unused): nothing unless
  // *gate != 0; N rows from *ncount (Np stays the layout's pitch)
  const int32_t* gate;
  const int32_t* ncount;
  int vec;                            // unit K stride, rows aligned for 4-element loads (k_predecode_w8)
};

// four consecutive elements of a row, k .. k+3 (k a multiple of 4): one
// 16-byte (f32) or 8-byte (bf16) load when all four lie within K, else one
// at a time with the elements past K zero
template <int DT>
__device__ __forceinline__ void load_elem4(const void* base, int64_t row_at, int64_t k, int64_t K, int64_t s_k,
                                           bool vec, uint32_t (&b)[4]) {
  if (vec && k + 4 <= K) {
    if (DT == DET_F32) {
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(base) + row_at + k);
      b[0] = v.x; b[1] = v.y; b[2] = v.z; b[3] = v.w;
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + row_at + k);
      b[0] = v.x & 0xFFFFu; b[1] = v.x >> 16; b[2] = v.y & 0xFFFFu; b[3] = v.y >> 16;
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) b[u] = k + u < K ? load_elem<DT>(base, row_at + (k + u) * s_k) : 0u;
  }
}

// Element i of a 32-bit array (layout [Kp/16][Np/64][4][64][4]) is (n, k);
// the 16-bit exponent array of k_gemm is [Kp/16][Np/64][2][64][8].
__device__ __forceinline__ void subblock_nk(int64_t i, int64_t np, int64_t& n, int64_t& k) {
  const int64_t c = i / (np * V_KC), r = i % (np * V_KC);
  const int64_t t = r / (V_BN * V_KC), r2 = r % (V_BN * V_KC);
  const int64_t q = r2 / (V_BN * 4), r3 = r2 % (V_BN * 4);
  n = t * V_BN + r3 / 4;
  k = c * V_KC + q * 4 + r3 % 4;
}
__device__ __forceinline__ int64_t exp16_index(int64_t n, int64_t k, int64_t np) {
  return (k / V_KC) * np * V_KC + (n / V_BN) * V_BN * V_KC + ((k % V_KC) / 8) * V_BN * 8 + (n % V_BN) * 8 + k % 8;
}

template <int DT, bool TWOS, uint32_t ESH, typename EW>
__global__ __launch_bounds__(256) void k_predecode_w(PredecodeArgs a) {
  static_assert(sizeof(EW) == 2, "k_gemm's exponent words are 16-bit");
  const int64_t total = a.Np * a.Kp;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  bool bad = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    int64_t n, k;
    subblock_nk(i, a.Np, n, k);
    int32_t m;
    uint32_t e;
    // padding holds the decode of +0 (significand 0, exponent field 1), so
    // the exponent sums of padded products stay inside the counter range
    const uint32_t b = n < a.N && k < a.K ? load_elem<DT>(a.w, n * a.w_sn + k * a.w_sk) : 0u;
    bad |= nonfinite_bits<DT>(b);
    decode<DT, TWOS, 1, ESH>(b, m, e);
    a.wsig[i] = m;
    static_cast<EW*>(a.wexp)[exp16_index(n, k, a.Np)] = static_cast<EW>(e);
  }
  note_nonfinite(bad);
}

// the same for k_gemm8: the grid's w-side words (32-bit), lane = n mod 64;
// block `blk` of `nblk` in a grid-stride loop
template <class G, int DT>
__device__ __forceinline__ void predecode_w8_body(PredecodeArgs a, int64_t blk, int64_t nblk) {
  if (a.gate != nullptr && *a.gate == 0) return;
  if (a.ncount != nullptr) a.N = *a.ncount;
  // with a device count only the chunks' first npd columns are decoded
  const int64_t npd = a.ncount != nullptr ? (a.N + V_BN - 1) / V_BN * V_BN : a.Np;
  const int64_t total = npd * a.Kp;
  const int64_t stride = nblk * blockDim.x;
  bool bad = false;
  if (a.vec) {
    // four consecutive words (one column, four consecutive k) per thread
    for (int64_t g = blk * blockDim.x + threadIdx.x; g < total / 4; g += stride) {
      const int64_t j = 4 * g;
      const int64_t i = npd == a.Np ? j : j / (npd * V_KC) * (a.Np * V_KC) + j % (npd * V_KC);
      int64_t n, k;
      subblock_nk(i, a.Np, n, k);
      uint32_t b[4] = {0u, 0u, 0u, 0u};
      if (n < a.N) load_elem4<DT>(a.w, (a.rmap != nullptr ? a.rmap[n] : n) * a.w_sn, k, a.K, a.w_sk, true, b);
      int32_t m[4];
      uint32_t e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bad |= nonfinite_bits<DT>(b[u]);
        G::decode_w(b[u], static_cast<uint32_t>(n & (V_BN - 1)), m[u], e[u]);
      }
      *reinterpret_cast<int4*>(a.wsig + i) = make_int4(m[0], m[1], m[2], m[3]);
      *reinterpret_cast<uint4*>(static_cast<uint32_t*>(a.wexp) + i) = make_uint4(e[0], e[1], e[2], e[3]);
    }
    note_nonfinite(bad);
    return;
  }
  for (int64_t j = blk * blockDim.x + threadIdx.x; j < total; j += stride) {
    const int64_t i = npd == a.Np ? j : j / (npd * V_KC) * (a.Np * V_KC) + j % (npd * V_KC);
    int64_t n, k;
    subblock_nk(i, a.Np, n, k);
    int32_t m;
    uint32_t e;
    const int64_t src = n < a.N && a.rmap != nullptr ? a.rmap[n] : n;
    const uint32_t b = n < a.N && k < a.K ? load_elem<DT>(a.w, src * a.w_sn + k * a.w_sk) : 0u;
    bad |= nonfinite_bits<DT>(b);
    G::decode_w(b, static_cast<uint32_t>(n & (V_BN - 1)), m, e);
    a.wsig[i] = m;
    static_cast<uint32_t*>(a.wexp)[i] = e;
  }
  note_nonfinite(bad);
}

template <class G, int DT>
__global__ __launch_bounds__(256) void k_predecode_w8(PredecodeArgs a) {
  predecode_w8_body<G, DT>(a, blockIdx.x, gridDim.x);
}

// x of one K block [M][K] (any strides) -> the x side's significands and
// words, [Mp][Kp] row-major with M padded to the tile's rows and K to the
// chunk, the padding holding the decode of +0; D::decode_x gives the words
// (D::ROWS rows per tile: row m is row m mod ROWS of its tile).
struct PredecodeXArgs {
  const void* x; int64_t x_sm, x_sk;
  int64_t M, K, Mp, Kp;
  int32_t* xsig; uint32_t* xword;
  const int32_t* rmap;                // decoded row m is row rmap[m] of x (null: m)
  // decided on the device (null: unused): nothing unless *gate != 0; M rows
  // from *mcount, padded to `mround`
  const int32_t* gate;
  const int32_t* mcount;
  int64_t mround;
  int vec;                            // unit K stride, rows aligned for 4-element loads
};


template <class D, int DT>
__device__ __forceinline__ void predecode_x_body(PredecodeXArgs a, int64_t blk, int64_t nblk) {
  if (a.gate != nullptr && *a.gate == 0) return;
  if (a.mcount != nullptr) {
    a.M = *a.mcount;
    a.Mp = (a.M + a.mround - 1) / a.mround * a.mround;
  }
  const int64_t total = a.Mp * a.Kp;
  const int64_t stride = nblk * blockDim.x;
  bool bad = false;
  if (a.vec) {
    // four consecutive k of one row per thread
    for (int64_t g = blk * blockDim.x + threadIdx.x; g < total / 4; g += stride) {
      const int64_t i = 4 * g, m = i / a.Kp, k = i % a.Kp;
      uint32_t b[4] = {0u, 0u, 0u, 0u};
      if (m < a.M) load_elem4<DT>(a.x, (a.rmap != nullptr ? a.rmap[m] : m) * a.x_sm, k, a.K, a.x_sk, true, b);
      int32_t v[4];
      uint32_t e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bad |= nonfinite_bits<DT>(b[u]);
        D::decode_x(b[u], static_cast<int>(m % D::ROWS), v[u], e[u]);
      }
      if constexpr (D::XPACK) {
        *reinterpret_cast<uint4*>(a.xsig + i) =
            make_uint4(D::pack_x(v[0], e[0]), D::pack_x(v[1], e[1]), D::pack_x(v[2], e[2]), D::pack_x(v[3], e[3]));
      } else {
        *reinterpret_cast<int4*>(a.xsig + i) = make_int4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<uint4*>(a.xword + i) = make_uint4(e[0], e[1], e[2], e[3]);
      }
    }
    note_nonfinite(bad);
    return;
  }
  for (int64_t i = blk * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t m = i / a.Kp, k = i % a.Kp;
    const int64_t src = m < a.M && a.rmap != nullptr ? a.rmap[m] : m;
    int32_t v;
    uint32_t e;
    const uint32_t b = m < a.M && k < a.K ? load_elem<DT>(a.x, src * a.x_sm + k * a.x_sk) : 0u;
    bad |= nonfinite_bits<DT>(b);
    D::decode_x(b, static_cast<int>(m % D::ROWS), v, e);
    if constexpr (D::XPACK) {
      a.xsig[i] = static_cast<int32_t>(D::pack_x(v, e));
    } else {
      a.xsig[i] = v;
      a.xword[i] = e;
    }
  }
  note_nonfinite(bad);
}

template <class D, int DT>
__global__ __launch_bounds__(256) void k_predecode_x(PredecodeXArgs a) {
  predecode_x_body<D, DT>(a, blockIdx.x, gridDim.x);
}

// both operands of a one-block k_gemm8 launch in one launch: blocks [0, nbw)
// decode w, the rest x
template <class G, int DT>
__global__ __launch_bounds__(256) void k_predecode_wx8(PredecodeArgs w, PredecodeXArgs x, int64_t nbw) {
  if (blockIdx.x < nbw) predecode_w8_body<G, DT>(w, blockIdx.x, nbw);
  else predecode_x_body<G, DT>(x, blockIdx.x - nbw, gridDim.x - nbw);
}

// the raw-digit kernel's x decode, in the form k_predecode_x takes
template <int DT, int R>
struct RawDecode {
  static constexpr int ROWS = R;
  static constexpr bool XPACK = false;
  __device__ static void decode_x(uint32_t b, int /*r*/, int32_t& m, uint32_t& e) {
    decode<DT, false, 0, EXP_SHIFT>(b, m, e);
  }
};

// ---------------------------------------------------------------- combine / finalize
struct CombineArgs {
  const int64_t* parts[COMBINE_MAX];
  int nparts;
  int64_t* out;
  int64_t n;                          // int64 elements
};

__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  bool bad = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < a.n; i += stride) {
    // a 128-bit sum: int64 partial sums may wrap although the total fits,
    // and wrapped sums may look in range although the total does not
    __int128 s = 0;
    for (int p = 0; p < a.nparts; ++p) {
      const int64_t v = a.parts[p][i];
      bad |= !digit_in_range(v);
      s += v;
    }
    const int64_t lo = static_cast<int64_t>(s);
    bad |= static_cast<__int128>(lo) != s || !digit_in_range(lo);
    a.out[i] = lo;
  }
  note_range(bad);
}

__global__ __launch_bounds__(256) void k_finalize(const int64_t* __restrict__ acc, float* __restrict__ y,
                                                   int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int64_t dg[ND];
  const int64_t* src = acc + i * ND;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    dg[j] = src[j];
    bad |= !digit_in_range(dg[j]);
  }
  note_range(bad);
  y[i] = __uint_as_float(round_digits_to_f32(dg));
}

__device__ __forceinline__ uint32_t round_bits_bf16(uint32_t b) {
  if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x7FFFFFu))
    return (b >> 16) | 0x40u;                                // NaN stays a (quiet) NaN
  // nearest-even on the bit pattern: add half an ulp minus one, plus the
  // lowest kept bit, then truncate; exact for every finite value and carries
  // into the exponent (up to Inf) where it must
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// VEC: 8 elements per thread (two 16-byte loads, one 16-byte store; both
// pointers 16-byte aligned), the last n mod 8 by the scalar form
template <bool VEC>
__global__ __launch_bounds__(256) void k_round_bf16(const uint32_t* __restrict__ in, uint16_t* __restrict__ out,
                                                     int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (VEC) {
    if (i >= n / 8) return;
    const uint4 a = reinterpret_cast<const uint4*>(in)[2 * i];
    const uint4 b = reinterpret_cast<const uint4*>(in)[2 * i + 1];
    reinterpret_cast<uint4*>(out)[i] =
        make_uint4(round_bits_bf16(a.x) | (round_bits_bf16(a.y) << 16), round_bits_bf16(a.z) | (round_bits_bf16(a.w) << 16),
                   round_bits_bf16(b.x) | (round_bits_bf16(b.y) << 16), round_bits_bf16(b.z) | (round_bits_bf16(b.w) << 16));
  } else {
    if (i >= n) return;
    out[i] = static_cast<uint16_t>(round_bits_bf16(in[i]));
  }
}

// The gradient of the mean squared error, elementwise: d = RNE32(y - t),
// gy = RNE32(RNE32(d * c) * g), dy = gy and dt = -gy in the operands' dtype
// (nearest-even for bf16).  Every fp32 operation is one IEEE operation, in
// this order, so the bits are those of the same expression evaluated one
// correctly rounded operation at a time.
template <int DT>
__device__ __forceinline__ float mse_load(const void* p, int64_t i) {
  if (DT == DET_F32) return static_cast<const float*>(p)[i];
  return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
}
template <int DT>
__device__ __forceinline__ void mse_store(void* p, int64_t i, float v) {
  if (DT == DET_F32) static_cast<float*>(p)[i] = v;
  else static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(round_bits_bf16(__float_as_uint(v)));
}
// eight consecutive elements (group q) with 16-byte accesses
template <int DT>
__device__ __forceinline__ void mse_load8(const void* p, int64_t q, float (&v)[8]) {
  if (DT == DET_F32) {
    const uint4 a = static_cast<const uint4*>(p)[2 * q], b = static_cast<const uint4*>(p)[2 * q + 1];
    const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(u[i]);
  } else {
    const uint4 a = static_cast<const uint4*>(p)[q];
    const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
}
template <int DT>
__device__ __forceinline__ void mse_store8(void* p, int64_t q, const float (&v)[8]) {
  if (DT == DET_F32) {
    static_cast<uint4*>(p)[2 * q] = make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                               __float_as_uint(v[3]));
    static_cast<uint4*>(p)[2 * q + 1] = make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]),
                                                   __float_as_uint(v[6]), __float_as_uint(v[7]));
  } else {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = round_bits_bf16(__float_as_uint(v[2 * i])) | (round_bits_bf16(__float_as_uint(v[2 * i + 1])) << 16);
    static_cast<uint4*>(p)[q] = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

// VEC: every operand 16-byte aligned; groups of eight elements with 16-byte
// accesses, then the last n mod 8 one at a time
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void k_mse_grad(const void* __restrict__ y, const void* __restrict__ t, int64_t n,
                                                   float c, const float* __restrict__ g, void* __restrict__ dy,
                                                   void* __restrict__ dt) {
  const float gv = *g;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t done = 0;
  if constexpr (VEC) {
    const int64_t groups = n / 8;
    for (int64_t q = first; q < groups; q += stride) {
      float d[8], gy[8], ng[8];
      mse_load8<DT>(y, q, d);
      if (t != nullptr) {
        float e[8];
        mse_load8<DT>(t, q, e);
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = __fsub_rn(d[i], e[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        gy[i] = __fmul_rn(__fmul_rn(d[i], c), gv);
        ng[i] = -gy[i];
      }
      if (dy != nullptr) mse_store8<DT>(dy, q, gy);
      if (dt != nullptr) mse_store8<DT>(dt, q, ng);
    }
    done = groups * 8;
  }
  for (int64_t i = done + first; i < n; i += stride) {
    float d = mse_load<DT>(y, i);
    if (t != nullptr) d = __fsub_rn(d, mse_load<DT>(t, i));
    const float gy = __fmul_rn(__fmul_rn(d, c), gv);
    if (dy != nullptr) mse_store<DT>(dy, i, gy);
    if (dt != nullptr) mse_store<DT>(dt, i, -gy);
  }
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
    if (DT == DET_F32) bad |= nonfinite_bits<DT>(static_cast<const uint32_t*>(p)[idx]);
    else bad |= nonfinite_bits<DT>(static_cast<const uint16_t*>(p)[idx]);
  }
  if (bad) *(flag != nullptr ? flag : &g_dev_status[0]) = 1;
}

// ---------------------------------------------------------------- det_gemm on the matrix cores
//
// det_gemm returns the exact sum rounded once, so how the exact sum is formed
// is free.  When the nonzero elements of every row of x and of w lie within a
// few binades of each other, it is formed with integer matrix products:
//   * a row is scaled by 2^-b (b = the row's top bit position + 3 - 8S), so
//     that each element becomes an integer V with |V| < 2^(8S-2), exactly as
//     long as the element's lowest set bit lies at or above b;
//   * V is cut into S balanced 8-bit digits, V = sum_s 2^(8s) V_s with V_s in
//     [-128, 127] (each digit is the sign-extended low byte of what remains);
//   * Z[i,j] = sum_k X[i,k] W[j,k] = sum_{s,t} 2^(8(s+t)) (X_s W_t^T)[i,j].
//     Each X_s W_t^T is an int8 GEMM on the MFMA units with int32 sums; the
//     products with the same s + t share one int32 sum over K blocks of
//     2^14 (|sum| <= 7 * 2^14 * 2^14 < 2^31), which are then added in
//     128-bit integers: |Z| < K 2^(16S-4) <= 2^127 for S <= 7, K <= 2^19;
//   * y[i,j] = RNE(Z[i,j] * 2^(bx[i] + bw[j])), the exact sum rounded once.
// A row of x (or of w) whose span needs more than S digits is recomputed on
// the exact-accumulator path after the matrix-core pass, which overwrites
// that row (column) of y; the pass's own values there are discarded.  The
// host picks S, or the accumulator path alone, from a histogram of the spans.

constexpr int SL_MIN = 2, SL_MAX = 7;     // digits per operand
constexpr int SL_KB = 64;                 // K per MFMA step
constexpr int64_t SL_FOLD = 256;          // MFMA steps (2^14 k) per int32 sum
constexpr int SL_TOP_NONE = -1000;        // top of an all-zero row
constexpr int SL_LOW_NONE = 1000;
constexpr int SL_HIST = 12;               // histogram bins per operand: need 0..8

// The plan of one call, made on the device from the span histogram (by the
// last workgroup of k_slice_need, or by k_slice_plan), and read by every
// later kernel of the call: int32 words in the workspace, behind the
// histograms.
constexpr int PL_S = 0;                   // digits per operand of the matrix-core pass; 0: the accumulator path
constexpr int PL_ACC = 1;                 // 1 when the accumulator path runs instead (its gate)
constexpr int PL_PREF = 2;                // the S the cost model prefers (0: the accumulator path)
constexpr int PL_TAILS = 3;               // 1: listed outputs keep their sums and get their tails added
constexpr int PL_FX = 4, PL_FW = 5;       // listed rows of x, of w
constexpr int PL_OX = 6, PL_OW = 7;       // rows of x, of w recomputed on the accumulator path
constexpr int PL_DONE = 8;                // workgroups of k_slice_need done (its last one makes the plan)
constexpr int PL_WORDS = 16;
constexpr int HP_WORDS = 2 * SL_HIST + PL_WORDS;   // the histograms and the plan, cleared by the span check

typedef int v4i __attribute__((ext_vector_type(4)));

// element bits -> sign, integer significand m and the exponent of its bit 0
// (value = +-m * 2^ex; subnormals keep their raw fraction)
template <int DT>
__device__ __forceinline__ void split_elem(uint32_t b, bool& neg, uint32_t& m, int& ex) {
  if (DT == DET_F32) {
    const uint32_t E = (b >> 23) & 0xFFu;
    m = (b & 0x7FFFFFu) | (min(E, 1u) << 23);
    ex = static_cast<int>(max(E, 1u)) - 150;
    neg = (b >> 31) != 0u;
  } else {
    const uint32_t E = (b >> 7) & 0xFFu;
    m = (b & 0x7Fu) | (min(E, 1u) << 7);
    ex = static_cast<int>(max(E, 1u)) - 134;
    neg = ((b >> 15) & 1u) != 0u;
  }
}

// Per row of an operand [R][K] (any strides): the top set bit position
// (max of ex + bit length - 1) and the lowest (min of ex + trailing zeros)
// over its nonzero elements, by atomic max / min into top[] and low[]
// (initialised to SL_TOP_NONE / SL_LOW_NONE).
constexpr int64_t STAT_KR = 4096;         // K elements per wave of the K-major span check

struct SliceStatArgs {
  const void* p; int64_t R, K, s_r, s_k;
  int32_t* top; int32_t* low;
  bool vec;                               // 16-byte loads: unit K stride and rows 16-byte aligned (K-major),
                                          // or unit row stride and 16-byte aligned columns (transposed)
  bool direct;                            // one wave (one thread) takes a whole row: store, no atomics
};

template <int DT>
__device__ __forceinline__ void stat_elem(uint32_t b, int& top, int& low, bool& bad) {
  bad |= nonfinite_bits<DT>(b);
  bool neg;
  uint32_t m;
  int ex;
  split_elem<DT>(b, neg, m, ex);
  if (m != 0u) {
    top = max(top, ex + 31 - __clz(static_cast<int>(m)));
    low = min(low, ex + __ffs(static_cast<int>(m)) - 1);
  }
}

// KMAJ (unit K stride): one wave per row and STAT_KR-element K range (four
// 1024-element parts, all of whose loads go out together), lanes along K;
// otherwise one thread per 256-element K range of one row (lanes along the
// rows, coalesced for a transposed view, 16 loads in flight), or with `vec`
// one block per 64 rows and 256-element K range, 16-byte loads along the rows
template <int DT, bool KMAJ>
__device__ __forceinline__ void stats_body(const SliceStatArgs& a, int64_t blk) {
  int top = SL_TOP_NONE, low = SL_LOW_NONE;
  bool bad = false;
  int64_t row;
  bool lead;
  if (KMAJ) {
    const int64_t nkr = (a.K + STAT_KR - 1) / STAT_KR;
    const int64_t wid = (blk * 256 + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (wid >= a.R * nkr) return;               // uniform per wave
    row = wid / nkr;
    const int64_t kr = (wid % nkr) * STAT_KR;
    constexpr int EPV = DT == DET_F32 ? 4 : 8;              // elements per 16-byte load
    if (a.vec && kr + STAT_KR <= a.K) {                      // lane: 16 consecutive elements per part
      uint4 v[STAT_KR / 1024][16 / EPV];
#pragma unroll
      for (int part = 0; part < STAT_KR / 1024; ++part) {
        const uint4* const q = reinterpret_cast<const uint4*>(
            static_cast<const char*>(a.p) + (row * a.s_r + kr + part * 1024 + lane * 16) * (DT == DET_F32 ? 4 : 2));
#pragma unroll
        for (int i = 0; i < 16 / EPV; ++i) v[part][i] = q[i];
      }
#pragma unroll
      for (int part = 0; part < STAT_KR / 1024; ++part)
#pragma unroll
        for (int i = 0; i < 16 / EPV; ++i) {
          const uint32_t w4[4] = {v[part][i].x, v[part][i].y, v[part][i].z, v[part][i].w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (DT == DET_F32) {
              stat_elem<DT>(w4[u], top, low, bad);
            } else {
              stat_elem<DT>(w4[u] & 0xFFFFu, top, low, bad);
              stat_elem<DT>(w4[u] >> 16, top, low, bad);
            }
          }
        }
    } else {
      for (int64_t k0 = kr; k0 < min(kr + STAT_KR, a.K); k0 += 1024) {
#pragma unroll 4
        for (int i = 0; i < 16; ++i) {
          const int64_t k = k0 + i * 64 + lane;
          if (k < a.K) stat_elem<DT>(load_elem<DT>(a.p, row * a.s_r + k), top, low, bad);
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      top = max(top, __shfl_xor(top, o));
      low = min(low, __shfl_xor(low, o));
    }
    lead = lane == 0;
  } else if (a.vec) {
    // rows contiguous and 16-byte aligned: a block takes 64 rows x 256 k;
    // thread t takes EPL consecutive rows (group t mod RG) and RG
    // consecutive k (one 16-byte load each); the threads of a row group
    // combine through shuffles, the waves through LDS, and one thread per
    // row stores it or adds it atomically
    constexpr int EPL = DT == DET_F32 ? 4 : 8, RG = 64 / EPL;
    constexpr int64_t ESZ = DT == DET_F32 ? 4 : 2;
    __shared__ int red[2][4][64];
    const int64_t nkr = (a.K + 255) / 256;
    const int64_t rb = blk / nkr, k0 = (blk % nkr) * 256;
    const int t = static_cast<int>(threadIdx.x), g = t % RG;
    const int64_t row0 = rb * 64 + g * EPL;
    const int64_t kq = k0 + (t / RG) * RG, k1 = min(kq + RG, a.K);
    int tops[EPL], lows[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) { tops[j] = SL_TOP_NONE; lows[j] = SL_LOW_NONE; }
    if (row0 + EPL <= a.R) {
      if (kq < k1) {
        uint4 q[RG];
#pragma unroll
        for (int u = 0; u < RG; ++u)          // clamped: a repeated element leaves max and min as they are
          q[u] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.p) +
                                                 (row0 + min(kq + u, k1 - 1) * a.s_k) * ESZ);
#pragma unroll
        for (int u = 0; u < RG; ++u) {
          const uint32_t w4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (DT == DET_F32) {
              stat_elem<DT>(w4[i], tops[i], lows[i], bad);
            } else {
              stat_elem<DT>(w4[i] & 0xFFFFu, tops[2 * i], lows[2 * i], bad);
              stat_elem<DT>(w4[i] >> 16, tops[2 * i + 1], lows[2 * i + 1], bad);
            }
          }
        }
      }
    } else {
      for (int64_t k = kq; k < k1; ++k)
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (row0 + j < a.R) stat_elem<DT>(load_elem<DT>(a.p, row0 + j + k * a.s_k), tops[j], lows[j], bad);
    }
    note_nonfinite(bad);
#pragma unroll
    for (int o = RG; o < 64; o <<= 1)
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        tops[j] = max(tops[j], __shfl_xor(tops[j], o));
        lows[j] = min(lows[j], __shfl_xor(lows[j], o));
      }
    const int wave = t >> 6;
    if ((t & 63) < RG) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        red[0][wave][g * EPL + j] = tops[j];
        red[1][wave][g * EPL + j] = lows[j];
      }
    }
    __syncthreads();
    if (t < 64 && rb * 64 + t < a.R) {
      const int top = max(max(red[0][0][t], red[0][1][t]), max(red[0][2][t], red[0][3][t]));
      const int low = min(min(red[1][0][t], red[1][1][t]), min(red[1][2][t], red[1][3][t]));
      if (a.direct) {
        a.top[rb * 64 + t] = top;
        a.low[rb * 64 + t] = low;
      } else if (top != SL_TOP_NONE) {
        atomicMax(a.top + rb * 64 + t, top);
        atomicMin(a.low + rb * 64 + t, low);
      }
    }
    return;
  } else {
    const int64_t t = blk * 256 + threadIdx.x;
    const int64_t nkr = (a.K + 255) / 256;
    if (t >= a.R * nkr) return;
    row = t % a.R;
    const int64_t k0 = (t / a.R) * 256, k1 = min(k0 + 256, a.K);
    for (int64_t kb = k0; kb < k1; kb += 16) {
      uint32_t e[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)            // clamped: a repeated element leaves max and min as they are
        e[u] = load_elem<DT>(a.p, row * a.s_r + min(kb + u, k1 - 1) * a.s_k);
#pragma unroll
      for (int u = 0; u < 16; ++u) stat_elem<DT>(e[u], top, low, bad);
    }
    lead = true;
  }
  note_nonfinite(bad);
  if (lead && a.direct) {                 // the row's only writer: no initial values needed
    a.top[row] = top;
    a.low[row] = low;
  } else if (lead && top != SL_TOP_NONE) {
    atomicMax(a.top + row, top);
    atomicMin(a.low + row, low);
  }
}

// x's and w's span check in one launch: blocks [0, nb0) take op[0], the
// rest op[1] (both operands need the same layout, KMAJ).  Block 0 also
// clears the histograms and the plan's words (k_slice_need fills them next).
struct SliceStatPair {
  SliceStatArgs op[2];
  int64_t nb0;
  int32_t* hist;
};

template <int DT, bool KMAJ>
__global__ __launch_bounds__(256) void k_slice_stats(SliceStatPair p) {
  const int64_t b = blockIdx.x;
  if (b == 0 && threadIdx.x < HP_WORDS && p.hist != nullptr) p.hist[threadIdx.x] = 0;   // the plan follows
  if (b < p.nb0) stats_body<DT, KMAJ>(p.op[0], b);
  else stats_body<DT, KMAJ>(p.op[1], b - p.nb0);
}

// initial tops and lows for rows that several waves share (atomics)
__global__ __launch_bounds__(256) void k_slice_init(int32_t* top, int32_t* low, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    top[i] = SL_TOP_NONE;
    low[i] = SL_LOW_NONE;
  }
}

// The choice between the paths: estimated seconds from the accumulator
// kernels' MAC rate and the int8 MAC rate of the slice pass (both measured
// on MI355X), S^2 int8 MACs per MAC plus the fallback rows and columns.
constexpr double RATE_ACC_F32 = 4.5e12, RATE_ACC_BF16 = 5.4e12, RATE_MMA = 1.2e15;
constexpr double SLICE_MIN_MACS = 134217728.0;    // 2^27: below, the accumulator path alone

// The plan of one call on the device, from the span histograms: the S the
// cost model prefers (the estimate above; `only`: no accumulator, `forced`:
// that S alone), the S the call runs (`mode` > 0: that one, fixed by the
// host; 0: the preferred one), the listed rows and whether their outputs
// keep their sums (at most `zfix` of them).  One thread.
struct PlanArgs {
  const int32_t* hist;                    // x's bins, then w's
  int32_t* plan;
  int64_t M, N, K, zfix;
  double rate_acc;
  int mode, only, forced;
};

__device__ void plan_body(const PlanArgs& a) {
  const int32_t* const hx = a.hist;
  const int32_t* const hw = a.hist + SL_HIST;
  const double macs = static_cast<double>(a.M) * a.N * a.K;
  double best = a.only ? 1e300 : macs / a.rate_acc;
  int pref = 0;
  for (int S = SL_MIN; S <= SL_MAX; ++S) {
    if (a.forced != 0 && S != a.forced) continue;
    int64_t cx = 0, cw = 0;
    for (int n = S + 1; n <= SL_MAX + 1; ++n) { cx += hx[n]; cw += hw[n]; }
    const double t = static_cast<double>(S) * S * macs / RATE_MMA +
                     (static_cast<double>(cx) * a.N * a.K + static_cast<double>(cw) * a.M * a.K) / a.rate_acc;
    if (t < best) { best = t; pref = S; }
  }
  const int run = a.mode > 0 ? a.mode : pref;
  int64_t fx = 0, fw = 0;
  if (run > 0)
    for (int n = run + 1; n <= SL_MAX + 1; ++n) { fx += hx[n]; fw += hw[n]; }
  const bool tails = run > 0 && fx + fw > 0 && fx * a.N + fw * a.M <= a.zfix;
  a.plan[PL_S] = run;
  a.plan[PL_ACC] = run == 0;
  a.plan[PL_PREF] = pref;
  a.plan[PL_TAILS] = tails;
  a.plan[PL_FX] = static_cast<int32_t>(fx);
  a.plan[PL_FW] = static_cast<int32_t>(fw);
  a.plan[PL_OX] = 0;
  a.plan[PL_OW] = 0;
}

__global__ __launch_bounds__(64) void k_slice_plan(PlanArgs a) {
  if (threadIdx.x == 0) plan_body(a);
}

// digits each row needs: the smallest S with top - low + 1 <= 8S - 2
// (0 for an all-zero row, 8 for more than SL_MAX), and their histograms
// (x's rows [0, split) count into hist[0..SL_HIST), w's rows after them into
// hist[SL_HIST..2 SL_HIST)); also clears the rows' tail counts
// With `fuse`, the last workgroup to finish makes the plan from the
// completed histograms (`pa`; the span check cleared the count of finished
// workgroups): one launch fewer per call.
__global__ __launch_bounds__(256) void k_slice_need(const int32_t* top, const int32_t* low, int64_t n,
                                                    int64_t split, int32_t* need, int32_t* hist, int32_t* cnt,
                                                    PlanArgs pa, int fuse) {
  __shared__ int32_t h[2 * SL_HIST];
  if (threadIdx.x < 2 * SL_HIST) h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int nd = top[i] == SL_TOP_NONE ? 0 : min((top[i] - low[i] + 10) / 8, SL_MAX + 1);
    need[i] = nd;
    cnt[i] = 0;
    atomicAdd(&h[(i < split ? 0 : SL_HIST) + nd], 1);
  }
  __syncthreads();
  if (threadIdx.x < 2 * SL_HIST && h[threadIdx.x] != 0) atomicAdd(hist + threadIdx.x, h[threadIdx.x]);
  if (!fuse) return;
  __threadfence();                        // this workgroup's histogram adds, before it counts itself done
  __syncthreads();
  if (threadIdx.x == 0 && atomicAdd(pa.plan + PL_DONE, 1) == static_cast<int>(gridDim.x) - 1) {
    __threadfence();                      // every other workgroup's adds are visible
    plan_body(pa);
  }
}

// list[] = the rows with need > S, in increasing order, and pos[r] = the
// place of row r in list[] or -1: workgroup 0 for x's M rows, workgroup 1 for
// w's N rows (w's arrays follow x's)
__global__ __launch_bounds__(1024) void k_slice_list(const int32_t* need, int64_t M, int64_t N, const int32_t* plan,
                                                     int32_t* list, int32_t* pos) {
  __shared__ int32_t wsum[16];
  __shared__ int64_t base;
  const int S = plan[PL_S];
  if (S == 0) return;
  const int64_t n = blockIdx.x == 0 ? M : N, at = blockIdx.x == 0 ? 0 : M;
  need += at;
  list += at;
  pos += at;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) base = 0;
  __syncthreads();
  for (int64_t r0 = 0; r0 < n; r0 += 1024) {
    const int64_t r = r0 + threadIdx.x;
    const bool flag = r < n && need[r] > S;
    const unsigned long long bal = __ballot(flag);
    const int pre = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int64_t off = base;
    for (int v = 0; v < wave; ++v) off += wsum[v];
    if (flag) list[off + pre] = static_cast<int32_t>(r);
    if (r < n) pos[r] = flag ? static_cast<int32_t>(off + pre) : -1;
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t t = base;
      for (int v = 0; v < 16; ++v) t += wsum[v];
      base = t;
    }
    __syncthreads();
  }
}

// ---- tails: the elements of a listed row below its window (lowest set bit
// under top + 3 - 8S), whose products the matrix-core pass leaves out
constexpr int SL_TAIL_CAP = 256;          // tails per row kept in a list; more: the row is recomputed
constexpr int64_t SL_ZFIX_MAX = int64_t(1) << 22;   // listed outputs whose 128-bit sums are kept

struct TailArgs {
  const void* p; int64_t K, s_r, s_k;     // the operand
  const int32_t* list;                    // its listed rows (plan[PL_FX + side] of them)
  const int32_t* top;
  const int32_t* plan; int side;          // side 0: x, 1: w
  int32_t* cnt;                           // tails per listed row
  int32_t* tk;                            // listed row p's first SL_TAIL_CAP tails' k at p * SL_TAIL_CAP
};

template <int DT>
__device__ __forceinline__ bool is_tail(uint32_t b, int base) {
  bool neg;
  uint32_t m;
  int ex;
  split_elem<DT>(b, neg, m, ex);
  return m != 0u && ex + __ffs(static_cast<int>(m)) - 1 < base;
}

// one wave per listed row and 1024-element K range: count the range's tails
// into the row's count (zeroed by k_slice_need) and write their k into the
// row's slot of tk at the places one atomic add reserved, as long as they
// fall within its first SL_TAIL_CAP (a row with more is recomputed whole,
// and the order of its tails does not matter to the exact sum)
template <int DT>
__device__ __forceinline__ void tail_scan_range(const TailArgs& a, int S, int64_t wid, int64_t nkr, int lane) {
  const int64_t p = wid / nkr, k0 = (wid % nkr) * 1024;
  const int64_t r = a.list[p];
  const int base = a.top[r] + 3 - 8 * S;
  uint32_t e[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t k = k0 + 64 * u + lane;
    e[u] = k < a.K ? load_elem<DT>(a.p, r * a.s_r + k * a.s_k) : 0u;
  }
  unsigned long long bal[16];
  int total = 0;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    bal[u] = __ballot(is_tail<DT>(e[u], base));
    total += __popcll(bal[u]);
  }
  if (total == 0) return;                                 // uniform per wave
  int at0 = 0;
  if (lane == 0) at0 = atomicAdd(a.cnt + p, total);
  int64_t c = __shfl(at0, 0);
  int32_t* const tk = a.tk + p * SL_TAIL_CAP;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int64_t at = c + __popcll(bal[u] & below);
    if (((bal[u] >> lane) & 1ull) && at < SL_TAIL_CAP) tk[at] = static_cast<int32_t>(k0 + 64 * u + lane);
    c += __popcll(bal[u]);
  }
}

// the listed rows' ranges, the waves of a capped grid taking them in turn
// (nothing when the plan keeps no tails)
// x's and w's tail scans in one launch: workgroups [0, nb0) take x
struct TailPair {
  TailArgs op[2];
  int64_t nb0;
};

template <int DT>
__global__ __launch_bounds__(256) void k_tail_scan(TailPair p) {
  const bool wside = blockIdx.x >= p.nb0;
  const TailArgs& a = p.op[wside ? 1 : 0];
  const int S = a.plan[PL_S];
  if (S == 0 || a.plan[PL_TAILS] == 0) return;
  const int64_t blk = wside ? blockIdx.x - p.nb0 : blockIdx.x, nb = wside ? gridDim.x - p.nb0 : p.nb0;
  const int64_t nkr = (a.K + 1023) / 1024, ranges = a.plan[PL_FX + a.side] * nkr;
  const int64_t waves = nb * 4;
  for (int64_t wid = (blk * 256 + threadIdx.x) >> 6; wid < ranges; wid += waves)
    tail_scan_range<DT>(a, S, wid, nkr, threadIdx.x & 63);
}

// off[p] = place of listed row p's tails in tk (its fixed slot; -1 for rows
// with more than SL_TAIL_CAP tails), ovl[] = the original indices of those
// rows, in order, and their count into the plan (one workgroup).  Without
// tails every listed row is recomputed.
__global__ __launch_bounds__(1024) void k_tail_plan(int32_t* plan, int64_t M, const int32_t* cnt, const int32_t* list,
                                                    int32_t* off, int32_t* ovl) {
  __shared__ int64_t wover[16];
  __shared__ int64_t obase;
  if (plan[PL_S] == 0) return;
  // workgroup 0: x's listed rows, workgroup 1: w's (w's arrays follow x's)
  const int side = blockIdx.x;
  const int64_t at = side == 0 ? 0 : M;
  cnt += at;
  list += at;
  off += at;
  ovl += at;
  const int64_t n = plan[PL_FX + side];
  if (plan[PL_TAILS] == 0) {
    for (int64_t p = threadIdx.x; p < n; p += 1024) ovl[p] = list[p];
    if (threadIdx.x == 0) plan[PL_OX + side] = static_cast<int32_t>(n);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) obase = 0;
  __syncthreads();
  for (int64_t p0 = 0; p0 < n; p0 += 1024) {
    const int64_t p = p0 + threadIdx.x;
    const bool over = p < n && cnt[p] > SL_TAIL_CAP;
    const unsigned long long bal = __ballot(over);
    if (lane == 0) wover[wave] = __popcll(bal);
    __syncthreads();
    int64_t ob = obase;
    for (int w = 0; w < wave; ++w) ob += wover[w];
    if (p < n) off[p] = over ? -1 : static_cast<int32_t>(p * SL_TAIL_CAP);
    if (over) ovl[ob + __popcll(bal & ((1ull << lane) - 1ull))] = list[p];
    __syncthreads();
    if (threadIdx.x == 0) {
      int64_t ot = obase;
      for (int w = 0; w < 16; ++w) ot += wover[w];
      obase = ot;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) plan[PL_OX + side] = static_cast<int32_t>(obase);
}

// dg += (-1)^neg * v * 2^(o - 298) for v < 2^128 (raw digits; the bits of
// v * 2^o below 2^0 must be zero)
__device__ __forceinline__ void add_u128(int64_t (&dg)[ND], bool neg, unsigned __int128 v, int o) {
  if (o < 0) { v = o > -128 ? v >> -o : 0; o = 0; }
  const int d = o >> 5, sh = o & 31;
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    const int bit = 32 * t - sh;                           // bit of v at the limb's bit 0
    uint64_t limb;
    if (bit < 0) limb = static_cast<uint64_t>(v << (-bit)) & 0xFFFFFFFFull;
    else limb = bit < 128 ? static_cast<uint64_t>(v >> bit) & 0xFFFFFFFFull : 0ull;
    if (limb != 0ull && d + t < ND) dg[d + t] += neg ? -static_cast<int64_t>(limb) : static_cast<int64_t>(limb);
  }
}

// dg += the exact product of two elements
template <int DT>
__device__ __forceinline__ void add_product(int64_t (&dg)[ND], uint32_t xb, uint32_t wb) {
  bool nx, nw;
  uint32_t mx, mw;
  int ex, ew;
  split_elem<DT>(xb, nx, mx, ex);
  split_elem<DT>(wb, nw, mw, ew);
  if (mx == 0u || mw == 0u) return;
  add_u128(dg, nx != nw, static_cast<unsigned __int128>(static_cast<uint64_t>(mx) * mw), ex + ew + 298);
}

// The listed outputs: row p of x's list with every column (zr, [nx][N]),
// then column q of w's list with every row not in x's list (zc, [nw][M]).
// Each adds its tail products to the matrix-core pass's exact sum Z and
// rounds once: y = RNE(Z 2^(bx + bw) + sum over x's tails k of x w + sum
// over w's tails k of x w where x[i,k] is not one of x's tails).  Rows
// and columns with off = -1 are left to the accumulator pass.
struct SliceFixArgs {
  const void* x; int64_t x_sm, x_sk;
  const void* w; int64_t w_sn, w_sk;
  int64_t M, N;
  int S;
  const int32_t* topx; const int32_t* topw;
  const int32_t* listx; const int32_t* listw;
  const int32_t* posx; const int32_t* posw;
  const int32_t* cntx; const int32_t* cntw;
  const int32_t* offx; const int32_t* offw;
  const int32_t* tkx; const int32_t* tkw;
  const int64_t* zr; const int64_t* zc;
  int64_t nx, nw;
  float* y; int64_t y_sm, y_sn;
  const int32_t* plan;                    // S, nx and nw are taken from the plan
};

template <int DT>
__global__ __launch_bounds__(256) void k_slice_fix(SliceFixArgs a) {
  a.S = a.plan[PL_S];
  if (a.S == 0 || a.plan[PL_TAILS] == 0) return;
  a.nx = a.plan[PL_FX];
  a.nw = a.plan[PL_FW];
  a.zc = a.zr + 2 * a.nx * a.N;                   // column sums follow the row sums
  const int64_t total = a.nx * a.N + a.nw * a.M;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total; t += stride) {
    int64_t i, j, p, q;
    const int64_t* zp;
    if (t < a.nx * a.N) {
      p = t / a.N;
      j = t % a.N;
      i = a.listx[p];
      q = a.posw[j];
      zp = a.zr + 2 * t;
    } else {
      const int64_t u = t - a.nx * a.N;
      q = u / a.M;
      i = u % a.M;
      p = a.posx[i];
      if (p >= 0) continue;                       // done with x's list
      j = a.listw[q];
      zp = a.zc + 2 * u;
    }
    if ((p >= 0 && a.offx[p] < 0) || (q >= 0 && a.offw[q] < 0)) continue;    // recomputed later
    const int bx = a.topx[i] + 3 - 8 * a.S, bw = a.topw[j] + 3 - 8 * a.S;
    int64_t dg[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) dg[d] = 0;
    const __int128 z = (static_cast<__int128>(zp[1]) << 64) | static_cast<__int128>(static_cast<uint64_t>(zp[0]));
    if (z != 0) {
      const bool neg = z < 0;
      add_u128(dg, neg, neg ? -static_cast<unsigned __int128>(z) : static_cast<unsigned __int128>(z), bx + bw + 298);
    }
    const int64_t xr = i * a.x_sm, wr = j * a.w_sn;
    if (p >= 0)
      for (int e = 0; e < a.cntx[p]; ++e) {
        const int64_t k = a.tkx[a.offx[p] + e];
        add_product<DT>(dg, load_elem<DT>(a.x, xr + k * a.x_sk), load_elem<DT>(a.w, wr + k * a.w_sk));
      }
    if (q >= 0)
      for (int e = 0; e < a.cntw[q]; ++e) {
        const int64_t k = a.tkw[a.offw[q] + e];
        const uint32_t xb = load_elem<DT>(a.x, xr + k * a.x_sk);
        if (p >= 0 && is_tail<DT>(xb, bx)) continue;          // counted with x's tails
        add_product<DT>(dg, xb, load_elem<DT>(a.w, wr + k * a.w_sk));
      }
    a.y[i * a.y_sm + j * a.y_sn] = __uint_as_float(round_digits_to_f32(dg));
  }
}

// The S digits of an operand [R][K], int8 in MFMA fragment order
// [Rb][Kb][S][64][16]: lane l, byte j of fragment (rb, kb, s) holds digit s of
// row 16 rb + (l mod 16), k = 64 kb + 16 (l div 16) + j, the A/B operand
// layout of v_mfma_i32_16x16x64_i8.  A wave loads one fragment as one
// contiguous KiB, and the S fragments of a step are adjacent.  Zero outside
// R x K, for zero elements and for elements below the row's window.  VEC:
// unit K stride with every 16-element run 16-byte aligned.
struct SliceMakeArgs {
  const void* p; int64_t R, K, s_r, s_k;
  const int32_t* top;
  int8_t* out;
  int64_t Rb, Kb;                     // 16-row and 64-k blocks (padded)
  int S;
  int vec;
};

// the S balanced 8-bit digits of 16 elements of one row (window bottom
// `base`), packed four to a word: digit s of element j in byte j mod 4 of
// d[s][j div 4]
template <int DT, typename V, int SMAX>
__device__ __forceinline__ void slice_digits_in(const uint32_t (&e)[16], int base, int S, uint32_t (&d)[SL_MAX][4]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    bool neg;
    uint32_t m;
    int ex;
    split_elem<DT>(e[j], neg, m, ex);
    const int sh = ex - base;
    if (m == 0u || sh + __ffs(static_cast<int>(m)) - 1 < 0) continue;    // zero, or below the window
    V v = sh >= 0 ? static_cast<V>(m) << sh : static_cast<V>(m >> (-sh));
    if (neg) v = -v;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      if (s < S) {
        const V dig = static_cast<int8_t>(static_cast<uint8_t>(v & 0xFF));
        v = (v - dig) >> 8;
        d[s][j >> 2] |= (static_cast<uint32_t>(dig) & 0xFFu) << (8 * (j & 3));
      }
    }
  }
}

// The same digits for S <= 4 (|V| < 2^30), four elements at a time: the
// balanced digits of V are the bytes of V + B, B = 0x80 in each of the S
// bytes, each less 128 (that is, with its top bit flipped), so the digit
// planes are a 4 x 4 byte transpose of the four words V + B (eight
// v_perm_b32) and one xor per word, in place of a shift-and-subtract per
// digit and element.
template <int DT>
__device__ __forceinline__ void slice_digits_perm(const uint32_t (&e)[16], int base, int S, uint32_t (&d)[SL_MAX][4]) {
  const uint32_t bias = S >= 4 ? 0x80808080u : 0x80808080u & ((1u << (8 * S)) - 1u);
  uint32_t u[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    bool neg;
    uint32_t m;
    int ex;
    split_elem<DT>(e[j], neg, m, ex);
    const int sh = ex - base;
    int32_t v = 0;
    if (m != 0u && sh + __ffs(static_cast<int>(m)) - 1 >= 0) {    // not zero, not below the window
      v = static_cast<int32_t>(sh >= 0 ? m << sh : m >> (-sh));
      if (neg) v = -v;
    }
    u[j] = static_cast<uint32_t>(v) + bias;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t* const w = u + 4 * q;
    const uint32_t t0 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);   // w0.b0 w1.b0 w0.b1 w1.b1
    const uint32_t t1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);   // w0.b2 w1.b2 w0.b3 w1.b3
    const uint32_t t2 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t t3 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    d[0][q] = __builtin_amdgcn_perm(t2, t0, 0x05040100u) ^ 0x80808080u;     // byte s of w0..w3
    d[1][q] = __builtin_amdgcn_perm(t2, t0, 0x07060302u) ^ 0x80808080u;
    if (S > 2) d[2][q] = __builtin_amdgcn_perm(t3, t1, 0x05040100u) ^ 0x80808080u;
    if (S > 3) d[3][q] = __builtin_amdgcn_perm(t3, t1, 0x07060302u) ^ 0x80808080u;
  }
}

// |V| < 2^(8S - 2): 32-bit arithmetic up to S = 4, 64-bit above
template <int DT>
__device__ __forceinline__ void slice_digits(const uint32_t (&e)[16], int base, int S, uint32_t (&d)[SL_MAX][4]) {
  if (S <= 4) slice_digits_perm<DT>(e, base, S, d);
  else slice_digits_in<DT, int64_t, SL_MAX>(e, base, S, d);
}

// fragment `blk` of the output, the lane's 16 bytes of each digit
__device__ __forceinline__ void slice_store(const SliceMakeArgs& a, int64_t blk, int lane,
                                            const uint32_t (&d)[SL_MAX][4]) {
#pragma unroll
  for (int s = 0; s < SL_MAX; ++s)
    if (s < a.S)
      *reinterpret_cast<uint4*>(a.out + ((blk * a.S + s) * 64 + lane) * 16) =
          make_uint4(d[s][0], d[s][1], d[s][2], d[s][3]);
}

template <int DT>
__device__ __forceinline__ void make_body(const SliceMakeArgs& a, int64_t blk, int64_t nblk) {
  const int64_t total = a.Rb * a.Kb * 64;
  const int64_t stride = nblk * blockDim.x;
  for (int64_t t = blk * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int lane = static_cast<int>(t & 63);
    const int64_t blk = t >> 6, rb = blk / a.Kb, kb = blk % a.Kb;
    const int64_t row = rb * 16 + (lane & 15), k0 = kb * 64 + (lane >> 4) * 16;
    uint32_t d[SL_MAX][4];
#pragma unroll
    for (int s = 0; s < SL_MAX; ++s) d[s][0] = d[s][1] = d[s][2] = d[s][3] = 0u;
    if (row < a.R) {
      const int base = a.top[row] + 3 - 8 * a.S;
      uint32_t e[16];
      if (a.vec && k0 + 16 <= a.K) {
        if (DT == DET_F32) {
          const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(a.p) + row * a.s_r + k0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 v = q[i];
            e[4 * i] = v.x; e[4 * i + 1] = v.y; e[4 * i + 2] = v.z; e[4 * i + 3] = v.w;
          }
        } else {
          const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.p) + row * a.s_r + k0);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint4 v = q[i];
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) { e[8 * i + 2 * u] = w4[u] & 0xFFFFu; e[8 * i + 2 * u + 1] = w4[u] >> 16; }
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          e[j] = k0 + j < a.K ? load_elem<DT>(a.p, row * a.s_r + (k0 + j) * a.s_k) : 0u;
      }
      slice_digits<DT>(e, base, a.S, d);
    }
    slice_store(a, blk, lane, d);
  }
}

// The same digits for an operand with unit row stride and K stride > 1 (a
// transposed view): a workgroup takes 64 rows (four 16-row blocks) by 64 k,
// reads them with the 64 rows along the lanes of a wave (one contiguous run
// per load), and hands each wave its block's elements through LDS.  The tile's rows are padded to 65 words,
// so the 16 k-runs a wave reads lie in four different bank quarters.
template <int DT>
__device__ __forceinline__ void make_t_body(const SliceMakeArgs& a, int64_t blk) {
  __shared__ uint32_t tile[64][65];
  const int64_t rb4 = blk / a.Kb, kb = blk % a.Kb;
  const int t = threadIdx.x;
  if (a.vec) {
    // 16-byte loads along the contiguous rows: EPL elements per load, LPK
    // lanes per k of the tile; rows past R (a partial load) element by element
    constexpr int EPL = DT == DET_F32 ? 4 : 8, LPK = 64 / EPL, KPP = 256 / LPK;
    constexpr int64_t ESZ = DT == DET_F32 ? 4 : 2;
    const int rg = (t % LPK) * EPL;
    const int64_t row0 = rb4 * 64 + rg;
#pragma unroll
    for (int pass = 0; pass < 64 / KPP; ++pass) {
      const int kl = pass * KPP + t / LPK;
      const int64_t k = kb * 64 + kl;
      uint32_t v[EPL];
      if (k < a.K && row0 + EPL <= a.R) {
        const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.p) + (row0 + k * a.s_k) * ESZ);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (DT == DET_F32) {
            v[j] = u[j];
          } else {
            v[2 * j] = u[j] & 0xFFFFu;
            v[2 * j + 1] = u[j] >> 16;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          v[j] = row0 + j < a.R && k < a.K ? load_elem<DT>(a.p, row0 + j + k * a.s_k) : 0u;
      }
#pragma unroll
      for (int j = 0; j < EPL; ++j) tile[kl][rg + j] = v[j];
    }
  } else {
    const int rl = t & 63, kq = t >> 6;                   // row of the tile (lane), quarter of its k
    const int64_t row = rb4 * 64 + rl;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kl = kq * 16 + i;
      const int64_t k = kb * 64 + kl;
      tile[kl][rl] = row < a.R && k < a.K ? load_elem<DT>(a.p, row + k * a.s_k) : 0u;
    }
  }
  __syncthreads();
  const int lane = t & 63, wave = t >> 6;
  const int rl = wave * 16 + (lane & 15), k0 = (lane >> 4) * 16;
  const int64_t rb = rb4 * 4 + wave, row = rb * 16 + (lane & 15);
  uint32_t d[SL_MAX][4];
#pragma unroll
  for (int s = 0; s < SL_MAX; ++s) d[s][0] = d[s][1] = d[s][2] = d[s][3] = 0u;
  if (row < a.R) {
    uint32_t e[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) e[j] = tile[k0 + j][rl];
    slice_digits<DT>(e, a.top[row] + 3 - 8 * a.S, a.S, d);
  }
  slice_store(a, rb * a.Kb + kb, lane, d);
}

// x's and w's digits in one launch: blocks [0, nb0) make op[0] (nb0 blocks),
// the rest op[1] (nb1)
struct SliceMakePair {
  SliceMakeArgs op[2];
  int64_t nb0, nb1;
  const int32_t* plan;                    // S is the plan's (nothing when it is 0)
};

template <int DT>
__global__ __launch_bounds__(256) void k_slice_make(SliceMakePair p) {
  p.op[0].S = p.op[1].S = p.plan[PL_S];
  if (p.op[0].S == 0) return;
  const int64_t b = blockIdx.x;
  if (b < p.nb0) make_body<DT>(p.op[0], b, p.nb0);
  else make_body<DT>(p.op[1], b - p.nb0, p.nb1);
}

template <int DT>
__global__ __launch_bounds__(256) void k_slice_make_t(SliceMakePair p) {
  p.op[0].S = p.op[1].S = p.plan[PL_S];
  if (p.op[0].S == 0) return;
  const int64_t b = blockIdx.x;
  if (b < p.nb0) make_t_body<DT>(p.op[0], b);
  else make_t_body<DT>(p.op[1], b - p.nb0);
}

// RNE(z * 2^e2) as binary32 bits (gradual underflow, overflow to inf; z = 0
// gives +0)
__device__ uint32_t round_i128_to_f32(__int128 z, int e2) {
  if (z == 0) return 0u;
  const bool neg = z < 0;
  const unsigned __int128 A = neg ? -static_cast<unsigned __int128>(z) : static_cast<unsigned __int128>(z);
  const uint64_t hi = static_cast<uint64_t>(A >> 64), lo = static_cast<uint64_t>(A);
  const int n = hi != 0u ? 127 - __clzll(static_cast<long long>(hi)) : 63 - __clzll(static_cast<long long>(lo));
  int q = max(n - 23, -149 - e2);                 // lowest kept bit of A
  uint32_t r;
  if (q <= 0) {
    r = static_cast<uint32_t>(A << (-q));         // exact: A < 2^(24 + q)
  } else if (q > 128) {
    r = 0u;                                       // |value| < 2^-150
  } else {
    const unsigned __int128 one = 1;
    const unsigned __int128 rr = q == 128 ? 0 : A >> q;
    const unsigned __int128 rem = q == 128 ? A : A & ((one << q) - 1);
    const unsigned __int128 half = one << (q - 1);
    r = static_cast<uint32_t>(rr);
    if (rem > half || (rem == half && (r & 1u))) r += 1u;
    if (r == (1u << 24)) { r = 1u << 23; q += 1; }
  }
  uint32_t mag;
  if (r < (1u << 23)) {
    mag = r;                                      // subnormal or zero: q + e2 == -149
  } else {
    const int E = q + e2 + 150;
    mag = E >= 255 ? 0x7F800000u : (static_cast<uint32_t>(E) << 23) | (r - (1u << 23));
  }
  return (neg ? 0x80000000u : 0u) | mag;
}

// The matrix-core pass (v_mfma_i32_16x16x64_i8).  A workgroup of 2 WR waves
// owns 32 WR rows x 32 CB columns; wave (wr, wc) owns 32 rows x 16 CB
// columns: 2 x CB blocks of 16 x 16, each with 2S-1 int32 sums (one per
// s + t).  Per 64-k step the workgroup's (2 WR + 2 CB) S fragments (one KiB
// each: 2 WR row blocks and 2 CB column blocks of x and w, S digits each) are
// copied from the digit arrays into one of NBUF LDS buffers with
// global_load_lds_dwordx4 (one instruction per fragment, no registers), NBUF
// - 1 steps ahead; each wave reads its 2S + CB S fragments from LDS, starts
// the copy of step kb + NBUF - 1 into the buffer read one step ago (the last
// ones repeat a step, so every copy is unconditional), and runs its 2 CB S^2
// MFMAs.  One barrier per step.  At most 256 registers per lane, so a SIMD
// switches between two waves while one reads LDS (two workgroups of 4 waves
// or one of 8 per CU; one wave for S = 7).  One launch covers at most 2^14
// k; longer K runs as several launches that carry each output's 128-bit sum
// in the workspace (epilogues as for the accumulator path).
struct SliceMmaArgs {
  const int8_t* xs; const int8_t* ws;
  int64_t Kb;                         // 64-k steps in the digit arrays
  int64_t kb0, kb1;                   // the steps of this launch
  int64_t M, N;
  int64_t tiles_m, tiles_n;
  const int32_t* topx; const int32_t* topw;
  float* y; int64_t y_sm, y_sn;
  int64_t* z;                         // 128-bit sums [M][N][2] (lo, hi) between launches
  int epi;
  // listed rows and columns, when the plan keeps tails: their final sums go
  // to zr [rows][N][2] (row in x's list) or zc [cols][M][2], not to y
  const int32_t* posx; const int32_t* posw;
  int64_t* zr; int64_t* zc;
  const int32_t* plan;                    // the launch does nothing unless the plan's S is this kernel's
};

template <int S, int CB, int WR, int NBUF>
struct SliceTile {
  static constexpr int NG = 2 * S - 1;
  static constexpr int NW = 2 * WR;             // waves
  static constexpr int FA = 2 * WR * S;         // x fragments per step
  static constexpr int FT = FA + 2 * CB * S;    // all fragments per step
  static constexpr int PER_WAVE = (FT + NW - 1) / NW;   // copies per wave (the last may be idle)
  static constexpr int LDS_BYTES = NBUF * FT * 1024;
};

// s_waitcnt with vmcnt(n) and the other counters left alone (gfx9 encoding)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Workgroup barrier without the release fence of __syncthreads (which would
// wait for every outstanding copy into LDS, including those a step or two
// ahead).  Callers first wait (vmcnt) for the copies the next step reads; the
// LDS reads of the step are complete, since its MFMAs consumed them.  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void step_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// this wave's copies of step kb into LDS buffer `buf`: fragment f = wave +
// NW j from src[j] (the lane's 16 bytes land at 16 * lane of the fragment)
template <class T>
__device__ __forceinline__ void slice_copy(const int8_t* const (&src)[T::PER_WAVE], int8_t* lds, int wave,
                                           int64_t kb, int buf, int64_t step_bytes) {
#pragma unroll
  for (int j = 0; j < T::PER_WAVE; ++j)
    if (T::FT % T::NW == 0 || j + 1 < T::PER_WAVE || wave + T::NW * j < T::FT)     // uniform per wave
      __builtin_amdgcn_global_load_lds(src[j] + kb * step_bytes, lds + buf * (T::FT * 1024) + (wave + T::NW * j) * 1024,
                                       16, 0, 0);
}

// one 64-k step: product (s, t) of block (i, c) into its sum for s + t.
// The lowest digit plane holds only the bits of elements far below their
// row's top, so its fragments are often all zero (on N(0,1) rows at S = 4,
// most of them): a product with such a fragment adds nothing and is skipped.
// The test is one ballot per fragment, uniform across the wave; a product
// that ran anyway would add zero, so the sums never depend on it.  At S = 7
// the branches cost more than they save (measured: 10 % slower), so that
// case keeps every product.
template <int S, int CB>
__device__ __forceinline__ void slice_steps(const v4i (&fa)[S][2], const v4i (&fb)[S][CB],
                                            v4i (&acc)[2 * S - 1][2][CB]) {
  constexpr bool SKIP = S <= 6;
  bool xa[2], wb[CB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    xa[i] = !SKIP || __ballot((fa[0][i].x | fa[0][i].y | fa[0][i].z | fa[0][i].w) != 0) != 0ull;
#pragma unroll
  for (int c = 0; c < CB; ++c)
    wb[c] = !SKIP || __ballot((fb[0][c].x | fb[0][c].y | fb[0][c].z | fb[0][c].w) != 0) != 0ull;
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int t = 0; t < S; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          if ((s == 0 && !xa[i]) || (t == 0 && !wb[c])) continue;
          acc[s + t][i][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[s][i], fb[t][c], acc[s + t][i][c], 0, 0, 0);
        }
}

// one workgroup's tile of the pass (`tile` in the XCD-aware order), with
// SliceTile<S, CB, WR, NBUF>::LDS_BYTES of LDS at `lds`
template <int S, int CB, int WR, int NBUF>
__device__ __forceinline__ void slice_mma_tile(SliceMmaArgs a, int8_t* lds, int64_t tile) {
  using T = SliceTile<S, CB, WR, NBUF>;
  constexpr int NG = T::NG, NW = T::NW, FA = T::FA, FT = T::FT, PW = T::PER_WAVE;
  const bool tails = a.plan[PL_TAILS] != 0;
  a.zc = a.zr + 2 * static_cast<int64_t>(a.plan[PL_FX]) * a.N;      // column sums follow the row sums
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  // tiles in groups of 8 rows of tiles, column by column within a group: the
  // workgroups resident on one XCD (consecutive in its range) cover about
  // 8 x 8 tiles, so each x and w fragment is fetched into that XCD's L2 once
  // for 8 workgroups
  const int64_t gsz = 8 * a.tiles_n, grp = tile / gsz, rows_g = min<int64_t>(8, a.tiles_m - 8 * grp);
  const int64_t tm = 8 * grp + (tile % gsz) % rows_g, tn = (tile % gsz) / rows_g;
  const int64_t rbw = 2 * WR * tm;                              // the workgroup's first 16-row block
  const int64_t cbw = 2 * CB * tn;                              // and first 16-column block
  const int64_t step_bytes = S * 1024;
  const int64_t fstep = a.Kb * step_bytes;                      // bytes between 16-row blocks

  // this wave copies fragments f = wave + NW j of every step: x block rbw + f
  // div S (f < FA) or w block cbw + (f - FA) div S, digit f mod S
  const int8_t* src[PW];
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    const int f = min(wave + NW * j, FT - 1);
    src[j] = f < FA ? a.xs + (rbw + f / S) * fstep + (f % S) * 1024
                    : a.ws + (cbw + (f - FA) / S) * fstep + ((f - FA) % S) * 1024;
    src[j] += lane * 16;
  }

  v4i acc[NG][2][CB];
#pragma unroll
  for (int u = 0; u < NG; ++u)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[u][i][c] = v4i{0, 0, 0, 0};

  // steps kb0 .. kb0 + NBUF - 2 in flight; wait for the first
  const int64_t last = a.Kb - 1;
#pragma unroll
  for (int b = 0; b + 1 < NBUF; ++b) slice_copy<T>(src, lds, wave, min(a.kb0 + b, last), b, step_bytes);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm((NBUF - 2) * PW));
  step_barrier();
  int buf = 0;
  for (int64_t kb = a.kb0; kb < a.kb1; ++kb) {
    const int8_t* const lb = lds + buf * (FT * 1024) + lane * 16;
    // this wave's fragments, in the order the MFMAs first use them
    v4i fa[S][2], fb[S][CB];
#pragma unroll
    for (int t = 0; t < S; ++t) {
      if (t == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[0][i] = *reinterpret_cast<const v4i*>(lb + ((2 * wr + i) * S) * 1024);
      }
#pragma unroll
      for (int c = 0; c < CB; ++c)
        fb[t][c] = *reinterpret_cast<const v4i*>(lb + (FA + (wc * CB + c) * S + t) * 1024);
    }
#pragma unroll
    for (int s = 1; s < S; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[s][i] = *reinterpret_cast<const v4i*>(lb + ((2 * wr + i) * S + s) * 1024);
    __builtin_amdgcn_sched_barrier(0);
    // into the buffer read one step ago (free since that step's barrier)
    const int nb = buf == 0 ? NBUF - 1 : buf - 1;
    slice_copy<T>(src, lds, wave, min(kb + NBUF - 1, last), nb, step_bytes);
    __builtin_amdgcn_sched_barrier(0);
    slice_steps<S, CB>(fa, fb, acc);
    __builtin_amdgcn_sched_barrier(0);                  // the wait and barrier stay behind the MFMAs
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NBUF - 2) * PW));   // this wave's copies of step kb + 1 landed
    step_barrier();                                      // everyone's, and buffer buf is free
    buf = buf + 1 == NBUF ? 0 : buf + 1;
  }

// output (row, col) of accumulator r of block (i, c): the MFMA's C layout
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int64_t col = (cbw + wc * CB + c) * 16 + (lane & 15);
    if (col >= a.N) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = (rbw + 2 * wr + i) * 16 + 4 * (lane >> 4) + r;
        if (row >= a.M) continue;
        __int128 z = 0;
#pragma unroll
        for (int u = 0; u < NG; ++u) z += static_cast<__int128>(acc[u][i][c][r]) << (8 * u);
        int64_t* const zp = a.z + (row * a.N + col) * 2;
        if (a.epi == EPI_ADD || a.epi == EPI_ADD_ROUND)
          z += (static_cast<__int128>(zp[1]) << 64) | static_cast<__int128>(static_cast<uint64_t>(zp[0]));
        int64_t* zo = nullptr;
        if (a.epi == EPI_STORE || a.epi == EPI_ADD) {
          zo = zp;
        } else if (tails) {
          const int32_t px = a.posx[row], pw = a.posw[col];
          if (px >= 0) zo = a.zr + (px * a.N + col) * 2;
          else if (pw >= 0) zo = a.zc + (static_cast<int64_t>(pw) * a.M + row) * 2;
        }
        if (zo != nullptr) {
          zo[0] = static_cast<int64_t>(z);
          zo[1] = static_cast<int64_t>(z >> 64);
        } else {
          const int e2 = (a.topx[row] + 3 - 8 * S) + (a.topw[col] + 3 - 8 * S);
          a.y[row * a.y_sm + col * a.y_sn] = __uint_as_float(round_i128_to_f32(z, e2));
        }
        asm volatile("" ::: "memory");          // one output at a time
      }
  }
}

template <int S, int CB, int WR, int NBUF>
__global__ __launch_bounds__(128 * WR, S >= 7 ? 1 : 2) void k_slice_mma(SliceMmaArgs a) {
  __shared__ __align__(16) int8_t lds[SliceTile<S, CB, WR, NBUF>::LDS_BYTES];
  if (a.plan[PL_S] != S) return;
  slice_mma_tile<S, CB, WR, NBUF>(a, lds, xcd_tile());
}

// Products of at most 512 tiles of 64 x 64 when the device's plan picks S:
// the shapes of S = 2 .. 6 in one launch (S = 7, which needs one workgroup
// per CU, keeps its own), so that the digit counts the plan did not pick
// cost one launch, not five.  Each shape is the narrow-tile one of
// launch_mma (16-column blocks halved), with the tile count of its own shape;
// the grid is the largest of them and the workgroups past a shape's count
// exit.
constexpr int SMALL_CB[8] = {0, 0, 2, 1, 1, 1, 1, 0};
constexpr int small_lds_bytes() {
  int m = 0;
  for (int S = 2; S <= 6; ++S) {
    const int b = 2 * (4 * S + 2 * SMALL_CB[S] * S) * 1024;
    m = b > m ? b : m;
  }
  return m;
}
constexpr int SMALL_LDS_BYTES = small_lds_bytes();

template <int S>
__device__ __forceinline__ void slice_mma_small(SliceMmaArgs a, int8_t* lds) {
  constexpr int CB = SMALL_CB[S];
  static_assert(SliceTile<S, CB, 2, 2>::LDS_BYTES <= SMALL_LDS_BYTES, "LDS");
  a.tiles_m = (a.M + 127) / 128 * 2;
  a.tiles_n = (a.N + 32 * CB - 1) / (32 * CB);
  const int64_t n = a.tiles_m * a.tiles_n;
  if (static_cast<int64_t>(blockIdx.x) >= n) return;
  slice_mma_tile<S, CB, 2, 2>(a, lds, xcd_tile_of(n));
}

__global__ __launch_bounds__(256, 2) void k_slice_mma_small(SliceMmaArgs a) {
  __shared__ __align__(16) int8_t lds[SMALL_LDS_BYTES];
  switch (a.plan[PL_S]) {
    case 2: slice_mma_small<2>(a, lds); break;
    case 3: slice_mma_small<3>(a, lds); break;
    case 4: slice_mma_small<4>(a, lds); break;
    case 5: slice_mma_small<5>(a, lds); break;
    case 6: slice_mma_small<6>(a, lds); break;
    default: break;
  }
}

// ---------------------------------------------------------------- exact dot products
//
// The raw digits of one long sum of exact products (det_dot_partial,
// det_sqdiff_partial): the reduction of a whole tensor into a single
// accumulator, e.g. a loss.  Each lane keeps two private sets of 18 int64
// slots in LDS, one slot per digit, for its positive and its negative
// products, and adds each product's base-2^32 limbs (three for f32, two for
// bf16) into the slots of the digits they fall in: one LDS atomic per limb,
// no contention (the slots are the lane's own) and no bank conflicts (a
// wave's 64 slots of one digit are 512 contiguous bytes and slot rows lie 512
// bytes apart, so the bank of a lane's slot depends on the lane alone).  The
// sign picks the set, so no limb is ever negated.  Every finite or
// non-finite bit pattern keeps its limbs within the 18 digits.  At the end
// the workgroup adds its lanes' slots digit by digit (positive minus
// negative) and adds each digit into the output with one 64-bit global
// atomic; integer addition is exact and commutative, so the digits do not
// depend on the order of the atomics.  The loop reads both operands once,
// 16 bytes per lane per load when they are contiguous and 16-byte aligned,
// with the next loads issued before the current elements are added: the
// kernel is bound by HBM bandwidth.

constexpr int DOT_W = 4;                  // waves per workgroup (two workgroups per CU)
constexpr int DOT_U = 4;                  // 16-byte loads per operand and lane per step
constexpr int DOT_SET = ND * 64;          // int64 slots of one sign of one wave
constexpr int64_t DOT_MAX_PRODUCTS = int64_t(1) << 30;

enum { DOT_PLAIN = 0, DOT_SQDIFF = 1, DOT_SQUARE = 2 };

struct DotArgs {
  const void* a; int64_t inc_a;
  const void* b; int64_t inc_b;
  int64_t n;
  int64_t* acc;                           // 18 digits
};

// an element as its integer significand and biased exponent max(E, 1): the
// value is +-m * 2^(Ez - 150) for f32, 2^(Ez - 134) for bf16
template <int DT>
__device__ __forceinline__ void dot_split(uint32_t b, uint32_t& m, uint32_t& ez) {
  if (DT == DET_F32) {
    const uint32_t E = (b >> 23) & 0xFFu;
    m = (b & 0x7FFFFFu) | (min(E, 1u) << 23);
    ez = max(E, 1u);
  } else {
    const uint32_t E = (b >> 7) & 0xFFu;
    m = (b & 0x7Fu) | (min(E, 1u) << 7);
    ez = max(E, 1u);
  }
}

// the product m1 * m2 * 2^(o - 298) added into the lane's slots of one sign;
// o >= 0 is the bit of the fixed-point accumulator that the product's bit 0
// lands on, `set` the lane's slot for digit 0 of that sign
template <int DT>
__device__ __forceinline__ void dot_add(unsigned long long* set, uint32_t m1, uint32_t m2, uint32_t o) {
  unsigned long long* const p = set + (o >> 5) * 64;
  const uint32_t sh = o & 31u;
  if (DT == DET_F32) {
    const uint64_t P = static_cast<uint64_t>(m1) * m2;                       // < 2^48
    const uint64_t lo = P << sh;                                             // limbs 0 and 1
    const uint32_t l2 = static_cast<uint32_t>(((P >> 32) << sh) >> 32);     // limb 2, < 2^15
    __hip_atomic_fetch_add(p, static_cast<unsigned long long>(static_cast<uint32_t>(lo)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_add(p + 64, static_cast<unsigned long long>(lo >> 32), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_add(p + 128, static_cast<unsigned long long>(l2), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    const uint64_t lo = static_cast<uint64_t>(m1 * m2) << sh;               // < 2^47: two limbs
    __hip_atomic_fetch_add(p, static_cast<unsigned long long>(static_cast<uint32_t>(lo)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_add(p + 64, static_cast<unsigned long long>(lo >> 32), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

// the products of one element pair (mode: a*b, (a-b)^2 = a*a + b*b - 2 a*b,
// or a*a); `pos` is the lane's positive set, the negative set follows it
template <int DT, int MODE>
__device__ __forceinline__ void dot_elem(unsigned long long* pos, uint32_t ab, uint32_t bb, bool& bad) {
  bad |= nonfinite_bits<DT>(ab);
  if (MODE != DOT_SQUARE) bad |= nonfinite_bits<DT>(bb);
  // o = (Ez_a - bias) + (Ez_b - bias) + 298: 298 - 300 for f32, 298 - 268 for bf16
  constexpr uint32_t OFF = DT == DET_F32 ? uint32_t(-2) : 30u;
  uint32_t ma, ea;
  dot_split<DT>(ab, ma, ea);
  if (MODE == DOT_SQUARE) {
    dot_add<DT>(pos, ma, ma, 2 * ea + OFF);
    return;
  }
  uint32_t mb, eb;
  dot_split<DT>(bb, mb, eb);
  const uint32_t sa = DT == DET_F32 ? ab >> 31 : (ab >> 15) & 1u;
  const uint32_t sb = DT == DET_F32 ? bb >> 31 : (bb >> 15) & 1u;
  if (MODE == DOT_PLAIN) {
    dot_add<DT>(pos + (sa ^ sb) * DOT_SET, ma, mb, ea + eb + OFF);
  } else {
    dot_add<DT>(pos, ma, ma, 2 * ea + OFF);
    dot_add<DT>(pos, mb, mb, 2 * eb + OFF);
    dot_add<DT>(pos + (1u ^ sa ^ sb) * DOT_SET, ma, mb, ea + eb + OFF + 1u);     // -2 a b
  }
}

// element e of a 16-byte load (4 f32 or 8 bf16 bit patterns); e is a
// compile-time index after unrolling
template <int DT>
__device__ __forceinline__ uint32_t dot_word_elem(const uint4& v, int e) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if (DT == DET_F32) return w[e];
  return (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
}

template <int DT, int MODE>
__device__ __forceinline__ void dot_load(const uint4* va, const uint4* vb, int64_t c, int64_t step, int64_t last,
                                         uint4 (&ra)[DOT_U], uint4 (&rb)[DOT_U]) {
#pragma unroll
  for (int u = 0; u < DOT_U; ++u) {
    const int64_t i = min(c + u * step, last);                   // clamped: always in bounds
    ra[u] = va[i];
    if (MODE != DOT_SQUARE) rb[u] = vb[i];
  }
}

template <int DT, int MODE, bool VEC>
__global__ __launch_bounds__(64 * DOT_W, 2) void k_dot(DotArgs a) {
  __shared__ unsigned long long slots[DOT_W * 2 * DOT_SET];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long* const pos = slots + wave * 2 * DOT_SET + lane;
#pragma unroll
  for (int j = 0; j < 2 * ND; ++j) pos[j * 64] = 0ull;
  // no barrier here: a lane touches only its own slots until the end
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  constexpr int EPV = DT == DET_F32 ? 4 : 8;         // elements per 16-byte load
  int64_t done = 0;
  bool bad = false;
  if (VEC) {
    const uint4* const va = static_cast<const uint4*>(a.a);
    const uint4* const vb = static_cast<const uint4*>(a.b);
    const int64_t nv = a.n / EPV, jump = nthreads * DOT_U;
    if (tid < nv) {
      uint4 ra[DOT_U], rb[DOT_U];
      dot_load<DT, MODE>(va, vb, tid, nthreads, nv - 1, ra, rb);
      for (int64_t c = tid; c < nv; c += jump) {
        uint4 na[DOT_U], nb[DOT_U];
        dot_load<DT, MODE>(va, vb, c + jump, nthreads, nv - 1, na, nb);
#pragma unroll
        for (int u = 0; u < DOT_U; ++u) {
          if (c + u * nthreads < nv) {
#pragma unroll
            for (int e = 0; e < EPV; ++e)
              dot_elem<DT, MODE>(pos, dot_word_elem<DT>(ra[u], e),
                                 MODE != DOT_SQUARE ? dot_word_elem<DT>(rb[u], e) : 0u, bad);
          }
        }
#pragma unroll
        for (int u = 0; u < DOT_U; ++u) { ra[u] = na[u]; rb[u] = nb[u]; }
      }
    }
    done = nv * EPV;
  }
  for (int64_t i = done + tid; i < a.n; i += nthreads) {
    const uint32_t x = load_elem<DT>(a.a, i * a.inc_a);
    const uint32_t y = MODE != DOT_SQUARE ? load_elem<DT>(a.b, i * a.inc_b) : 0u;
    dot_elem<DT, MODE>(pos, x, y, bad);
  }
  note_nonfinite(bad);
  __syncthreads();
  // digit j: lane l adds slot j of lane l of every wave (positive minus
  // negative), then the wave adds its 64 lanes
  for (int j = wave; j < ND; j += DOT_W) {
    int64_t s = 0;
#pragma unroll
    for (int w = 0; w < DOT_W; ++w) {
      const unsigned long long* const q = slots + w * 2 * DOT_SET + j * 64 + lane;
      s += static_cast<int64_t>(q[0]) - static_cast<int64_t>(q[DOT_SET]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0 && s != 0)
      __hip_atomic_fetch_add(reinterpret_cast<unsigned long long*>(a.acc + j), static_cast<unsigned long long>(s),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ __launch_bounds__(64) void k_zero_digits(int64_t* acc) {
  if (threadIdx.x < ND) acc[threadIdx.x] = 0;
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

template <int DT, int MODE>
void launch_dot(const DotArgs& a, bool vec, hipStream_t s) {
  constexpr int EPV = DT == DET_F32 ? 4 : 8;
  const int64_t per_block = static_cast<int64_t>(64) * DOT_W * (vec ? EPV * DOT_U : 4);
  const dim3 grid(grid_for(a.n, per_block, 512)), block(64 * DOT_W);     // two per CU
  if (vec) hipLaunchKernelGGL((k_dot<DT, MODE, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((k_dot<DT, MODE, false>), grid, block, 0, s, a);
}

det_status dot_common(int mode, det_dtype dt, const void* a, int64_t inc_a, const void* b, int64_t inc_b,
                      int64_t n, int64_t* acc, int accumulate, void* stream) {
  if (dt != DET_F32 && dt != DET_BF16) return fail(DET_EDTYPE, "unknown dtype %d", static_cast<int>(dt));
  if (n < 0 || inc_a < 0 || inc_b < 0) return fail(DET_EINVAL, "negative count or increment");
  const int64_t per = mode == DOT_SQDIFF ? 3 : 1;
  if (n > DOT_MAX_PRODUCTS / per)
    return fail(DET_EKLIMIT, "%lld elements exceed the limit of 2^30 products per accumulator", (long long)n);
  if (acc == nullptr) return fail(DET_EINVAL, "null accumulator");
  if (reinterpret_cast<uintptr_t>(acc) & 7u) return fail(DET_EINVAL, "accumulator must be 8-byte aligned");
  if (n > 0 && (a == nullptr || (mode != DOT_SQUARE && b == nullptr))) return fail(DET_EINVAL, "null operand");
  const uintptr_t align = dt == DET_F32 ? 4u : 2u;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & (align - 1))
    return fail(DET_EINVAL, "operands must be aligned to their element size");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!accumulate) {
    hipLaunchKernelGGL(k_zero_digits, dim3(1), dim3(64), 0, s, acc);
    det_status st = hip_check(hipGetLastError(), "dot zero launch");
    if (st != DET_OK) return st;
  }
  if (n == 0) return DET_OK;
  DotArgs d{a, inc_a, mode == DOT_SQUARE ? a : b, mode == DOT_SQUARE ? inc_a : inc_b, n, acc};
  const bool vec = d.inc_a == 1 && d.inc_b == 1 &&
                   ((reinterpret_cast<uintptr_t>(d.a) | reinterpret_cast<uintptr_t>(d.b)) & 15u) == 0u;
  if (dt == DET_F32) {
    if (mode == DOT_PLAIN) launch_dot<DET_F32, DOT_PLAIN>(d, vec, s);
    else if (mode == DOT_SQDIFF) launch_dot<DET_F32, DOT_SQDIFF>(d, vec, s);
    else launch_dot<DET_F32, DOT_SQUARE>(d, vec, s);
  } else {
    if (mode == DOT_PLAIN) launch_dot<DET_BF16, DOT_PLAIN>(d, vec, s);
    else if (mode == DOT_SQDIFF) launch_dot<DET_BF16, DOT_SQDIFF>(d, vec, s);
    else launch_dot<DET_BF16, DOT_SQUARE>(d, vec, s);
  }
  return hip_check(hipGetLastError(), "dot launch");
}

// K per launch.  With a longer K range the waves resident on one XCD drift
// apart in k and stop sharing their slice of w in L2 (measured: 2400 GMAC/s at
// K = 2^15, 824 at K = 2^19 in one launch), so longer ranges run as several
// launches of this length that carry the exact digits between them.
constexpr int64_t K_BLOCK = int64_t(1) << 15;

// workspace: the pre-decoded w, the pre-decoded x of one K block (8 bytes
// per element, rows padded to 2, K to 16), then (det_gemm with K > K_BLOCK)
// int64 digit scratch for the output.  det_gemm's kernel takes 32-bit
// exponent words for w, the partial's 16-bit ones.
constexpr int TILE_ROWS = 2;
int64_t predecode_bytes(int out_mode, int64_t N, int64_t K) {
  return round_up(N, V_BN) * round_up(K, V_KC) * (out_mode == 1 ? 4 + 4 : 4 + 2);
}
int64_t xdecode_bytes(int64_t M, int64_t K) {
  return round_up(M, TILE_ROWS) * round_up(min(K, K_BLOCK), V_KC) * (4 + 4);
}
int64_t workspace_bytes(int out_mode, int64_t M, int64_t N, int64_t K) {
  int64_t b = predecode_bytes(out_mode, N, K) + xdecode_bytes(M, K);
  if (out_mode == 1 && K > K_BLOCK) b += M * N * ND * 8;
  return b;
}

// the decode of x's K block [k0, k0 + kb) into the workspace region at
// `xr` (b.K = kb), and b's pointers to it
PredecodeXArgs x_decode_args(GemmArgs& b, const void* xblock, char* xr, int64_t esz) {
  PredecodeXArgs p{};
  p.x = xblock; p.x_sm = b.x_sm; p.x_sk = b.x_sk;
  p.M = b.M; p.K = b.K; p.Mp = round_up(b.M, TILE_ROWS); p.Kp = round_up(b.K, V_KC);
  p.xsig = reinterpret_cast<int32_t*>(xr);
  p.xword = reinterpret_cast<uint32_t*>(xr + p.Mp * p.Kp * 4);
  p.rmap = b.xmap;
  p.gate = b.gate; p.mcount = b.mcount; p.mround = TILE_ROWS;
  p.vec = b.x_sk == 1 && reinterpret_cast<uintptr_t>(xblock) % (4 * esz) == 0 && (b.x_sm * esz) % (4 * esz) == 0;
  b.xsig = p.xsig; b.xword = p.xword; b.xld = p.Kp;
  return p;
}

template <class D, int DT>
det_status predecode_x_block(GemmArgs& b, const void* xblock, char* xr, hipStream_t s) {
  const PredecodeXArgs p = x_decode_args(b, xblock, xr, DT == DET_F32 ? 4 : 2);
  hipLaunchKernelGGL((k_predecode_x<D, DT>), dim3(grid_for(p.Mp * p.Kp / (p.vec ? 4 : 1), 256, 8192)), dim3(256), 0,
                     s, p);
  return hip_check(hipGetLastError(), "x predecode launch");
}

// Raw digits (det_gemm_partial): k_partial with 64 columns per workgroup of
// 4 waves (50 KB of counters, three workgroups per CU, 3 waves per SIMD).
// f32 takes one row per workgroup with the 64-bit pair counters (two LDS
// atomics per product instead of four; measured 8-12 % faster), bf16 two
// rows with 32-bit counters (its products have two fields, and the second row
// that reuses each w element matters more: the pair form was 10 % slower).
// K runs in blocks of 2^15, with or without a workspace, so no counter can
// overflow; the digits are carried in acc.
// Without a workspace the GEMM kernels decode x and w themselves and no
// pre-decode pass sees every element once: one checking pass per operand
// notes an Inf or NaN in the device status instead.
template <int DT>
det_status note_raw_operands(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_check_finite<DT>, dim3(grid_for(a.M * a.K, 256, 4096)), dim3(256), 0, s, a.x, a.M, a.K, a.x_sm,
                     a.x_sk, nullptr);
  hipLaunchKernelGGL(k_check_finite<DT>, dim3(grid_for(a.N * a.K, 256, 4096)), dim3(256), 0, s, a.w, a.N, a.K, a.w_sn,
                     a.w_sk, nullptr);
  return hip_check(hipGetLastError(), "operand check launch");
}

template <int DT>
det_status launch_partial(GemmArgs a, void* ws, hipStream_t s) {
  constexpr bool PAIR = DT == DET_F32;
  constexpr int R = PAIR ? 1 : 2, W = 4, WPE = 3;
  a.tiles_m = (a.M + R - 1) / R;
  a.tiles_n = (a.N + V_BN - 1) / V_BN;
  const int64_t blocks = a.tiles_m * a.tiles_n;
  if (blocks == 0) return DET_OK;
  if (blocks > 0x7FFFFFFF) return fail(DET_EINVAL, "too many output tiles");
  // 16-byte vector loads of w chunks: unit K-stride and every chunk start aligned
  const int64_t esz = DT == DET_F32 ? 4 : 2;
  a.w_vec = a.w_sk == 1 && (reinterpret_cast<uintptr_t>(a.w) % 16) == 0 && (a.w_sn * esz) % 16 == 0;
  const bool pre = ws != nullptr && a.K > 0;
  if (!pre && a.K > 0) {
    det_status st = note_raw_operands<DT>(a, s);
    if (st != DET_OK) return st;
  }
  if (pre) {
    PredecodeArgs p{};
    p.w = a.w; p.w_sn = a.w_sn; p.w_sk = a.w_sk;
    p.N = a.N; p.K = a.K; p.Np = round_up(a.N, V_BN); p.Kp = round_up(a.K, V_KC);
    p.wsig = static_cast<int32_t*>(ws);
    p.wexp = static_cast<char*>(ws) + p.Np * p.Kp * 4;
    a.wsig = p.wsig; a.wexp = static_cast<const uint16_t*>(p.wexp); a.wld = p.Np * V_KC;
    const dim3 pg(grid_for(p.Np * p.Kp, 256, 8192));
    hipLaunchKernelGGL((k_predecode_w<DT, false, EXP_SHIFT, uint16_t>), pg, dim3(256), 0, s, p);
    det_status st = hip_check(hipGetLastError(), "predecode launch");
    if (st != DET_OK) return st;
  }
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * W);
  const int64_t nblk = a.K > 0 ? (a.K + K_BLOCK - 1) / K_BLOCK : 1;
  for (int64_t ib = 0; ib < nblk; ++ib) {
    GemmArgs b = a;
    const int64_t k0 = ib * K_BLOCK;
    b.K = min(K_BLOCK, a.K - k0);
    const void* xb = static_cast<const char*>(a.x) + k0 * a.x_sk * esz;
    const void* wb = static_cast<const char*>(a.w) + k0 * a.w_sk * esz;
    // raw w of this block: alignment of its chunk starts as for the whole w
    b.w = wb;
    b.w_vec = a.w_vec && (reinterpret_cast<uintptr_t>(wb) % 16) == 0;
    if (pre) { b.wsig = a.wsig + k0 / V_KC * a.wld; b.wexp = a.wexp + k0 / V_KC * a.wld; }
    b.epi = ib == 0 ? EPI_STORE : EPI_ADD;
    if (pre) {
      det_status st = predecode_x_block<RawDecode<DT, R>, DT>(
          b, xb, static_cast<char*>(ws) + predecode_bytes(0, a.N, a.K), s);
      if (st != DET_OK) return st;
    }
    det_status st = mark_event(g_ev_start, ib == 0, s);
    if (st != DET_OK) return st;
    if (pre) hipLaunchKernelGGL((k_partial<DT, true, R, PAIR, W, WPE>), grid, block, 0, s, b, xb, wb);
    else hipLaunchKernelGGL((k_partial<DT, false, R, PAIR, W, WPE>), grid, block, 0, s, b, xb, wb);
    st = hip_check(hipGetLastError(), "gemm launch");
    if (st == DET_OK) st = mark_event(g_ev_stop, ib + 1 == nblk, s);
    if (st != DET_OK) return st;
  }
  return DET_OK;
}

// det_gemm: k_gemm8's configuration per dtype: rows per workgroup, waves,
// waves per SIMD and the cell grid.  f32: the 4-bit grid (4096 adds between
// folds) on 2 rows, 128 KB of cells shared by 16 waves, one workgroup per CU:
// 3655 GMAC/s on the wide-range 4096^3 workload when it was chosen, against
// 3465 for the 8-bit grid (64 KB, 8 waves, two workgroups per CU), 3373 for
// the 4-bit grid on one row, and 3231 for a 4-bit grid with the shift split
// between the operands at decode (three VALU instructions per product instead
// of six, but 27-bit operands leave 512 adds between folds: the LDS, not the
// VALU, binds).  bf16 keeps two 64 KB workgroups of 8 waves (four rows on 128
// KB: 4570 against 5369).
constexpr int64_t GEMM8_LIST_GRID = 1024;    // workgroups of a device-counted recompute
constexpr int64_t GEMM8_LOOP_TPW = 32;       // most tiles per workgroup of a looping launch
constexpr int64_t GEMM8_LOOP_GRID = 2048;    // fewest workgroups a looping launch keeps

template <int DT> struct Gemm8Config;
template <> struct Gemm8Config<DET_F32> {
  static constexpr int R = 2, W = 16, WPE = 4;
  using G = CellsG<DET_F32, R, 4>;
};
template <> struct Gemm8Config<DET_BF16> {
  static constexpr int R = 2, W = 8, WPE = 4;
  using G = Cells4<R>;
};

template <int DT>
det_status launch_gemm8(GemmArgs a, void* ws, hipStream_t s, int marks = MARK_BOTH) {
  using C = Gemm8Config<DT>;
  constexpr int R = C::R, W = C::W, WPE = C::WPE;
  using G = typename C::G;
  a.tiles_m = (a.M + R - 1) / R;
  a.tiles_n = (a.N + V_BN - 1) / V_BN;
  const int64_t blocks = a.tiles_m * a.tiles_n;
  if (blocks == 0) return DET_OK;
  if (blocks > 0x7FFFFFFF) return fail(DET_EINVAL, "too many output tiles");
  const int64_t esz = DT == DET_F32 ? 4 : 2;
  a.w_vec = a.w_sk == 1 && (reinterpret_cast<uintptr_t>(a.w) % 16) == 0 && (a.w_sn * esz) % 16 == 0;
  const bool pre = ws != nullptr && a.K > 0;
  const bool listed = a.mcount != nullptr || a.ncount != nullptr;
  if (!pre && a.K > 0 && !listed) {               // (listed rows' operands were checked by the span check)
    det_status st = note_raw_operands<DT>(a, s);
    if (st != DET_OK) return st;
  }
  // K blocks; beyond one block the exact digits are carried in the
  // workspace, behind the decoded w
  const int64_t kblk = pre ? K_BLOCK : a.K;
  const int64_t nblk = a.K > 0 ? (a.K + kblk - 1) / kblk : 1;
  if (pre) {
    PredecodeArgs p{};
    p.w = a.w; p.w_sn = a.w_sn; p.w_sk = a.w_sk;
    p.N = a.N; p.K = a.K; p.Np = round_up(a.N, V_BN); p.Kp = round_up(a.K, V_KC);
    p.wsig = static_cast<int32_t*>(ws);
    p.wexp = static_cast<char*>(ws) + p.Np * p.Kp * 4;
    a.wsig = p.wsig; a.wexp32 = static_cast<const uint32_t*>(p.wexp); a.wld = p.Np * V_KC;
    p.rmap = a.wmap;
    p.gate = a.gate; p.ncount = a.ncount;
    p.vec = a.w_sk == 1 && reinterpret_cast<uintptr_t>(a.w) % (4 * esz) == 0 && (a.w_sn * esz) % (4 * esz) == 0;
    const int64_t nbw = grid_for(p.Np * p.Kp / (p.vec ? 4 : 1), 256, 8192);
    if (nblk == 1) {                              // x's only K block with w, in one launch
      const PredecodeXArgs px = x_decode_args(a, a.x, static_cast<char*>(ws) + predecode_bytes(1, a.N, a.K), esz);
      const int64_t nbx = grid_for(px.Mp * px.Kp / (px.vec ? 4 : 1), 256, 8192);
      hipLaunchKernelGGL((k_predecode_wx8<G, DT>), dim3(static_cast<unsigned>(nbw + nbx)), dim3(256), 0, s, p, px,
                         nbw);
    } else {
      hipLaunchKernelGGL((k_predecode_w8<G, DT>), dim3(static_cast<unsigned>(nbw)), dim3(256), 0, s, p);
    }
    det_status st = hip_check(hipGetLastError(), "predecode launch");
    if (st != DET_OK) return st;
  }
  // The looping form (consecutive tiles per workgroup) for the work the
  // device decides (a gate, device-counted rows or columns) and for every
  // pre-decoded launch of the claiming (f32) kernel, whose tiles after a
  // workgroup's first neither clear LDS nor wait for a rounding.  Tiles per
  // workgroup: a capped grid for device-counted rows or columns, else up to
  // GEMM8_LOOP_TPW, keeping eight workgroups per CU where the tiles allow.
  if (a.gate != nullptr && !listed && !pre) return fail(DET_EINVAL, "a gated launch needs the workspace");
  const bool loop = listed || a.gate != nullptr || (G::CLAIM && pre);
  a.tpw = listed ? (blocks + GEMM8_LIST_GRID - 1) / GEMM8_LIST_GRID
         : loop   ? std::max<int64_t>(1, std::min(GEMM8_LOOP_TPW, blocks / GEMM8_LOOP_GRID))
                  : 1;
  const dim3 grid(static_cast<unsigned>((blocks + a.tpw - 1) / a.tpw)), block(64 * W);
  if (nblk > 1)
    a.acc = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + predecode_bytes(1, a.N, a.K) +
                                       xdecode_bytes(a.M, a.K));
  for (int64_t ib = 0; ib < nblk; ++ib) {
    GemmArgs b = a;
    const int64_t k0 = ib * kblk;
    b.K = min(kblk, a.K - k0);
    const void* xb = static_cast<const char*>(a.x) + k0 * a.x_sk * esz;
    if (pre) { b.wsig = a.wsig + k0 / V_KC * a.wld; b.wexp32 = a.wexp32 + k0 / V_KC * a.wld; }
    const bool first = ib == 0, last = ib + 1 == nblk;
    b.epi = nblk == 1 ? EPI_ROUND : first ? EPI_STORE : last ? EPI_ADD_ROUND : EPI_ADD;
    if (pre && nblk > 1) {
      det_status st = predecode_x_block<G, DT>(b, xb, static_cast<char*>(ws) + predecode_bytes(1, a.N, a.K), s);
      if (st != DET_OK) return st;
    }
    det_status st = mark_event(g_ev_start, (marks & MARK_START) && first, s);
    if (st != DET_OK) return st;
    if (loop && !pre) {
      hipLaunchKernelGGL((k_gemm8<G, DT, false, R, W, WPE, true>), grid, block, 0, s, b, xb, a.w);
    } else if (loop) {
      hipLaunchKernelGGL((k_gemm8<G, DT, true, R, W, WPE, true>), grid, block, 0, s, b, xb, a.w);
    } else if (!pre) {
      hipLaunchKernelGGL((k_gemm8<G, DT, false, R, W, WPE, false>), grid, block, 0, s, b, xb, a.w);
    } else if constexpr (!G::CLAIM) {
      hipLaunchKernelGGL((k_gemm8<G, DT, true, R, W, WPE, false>), grid, block, 0, s, b, xb, a.w);
    }
    st = hip_check(hipGetLastError(), "gemm launch");
    if (st == DET_OK) st = mark_event(g_ev_stop, (marks & MARK_STOP) && last, s);
    if (st != DET_OK) return st;
  }
  return DET_OK;
}

// ---------------------------------------------------------------- det_gemm: the matrix-core path
//
// Workspace behind the accumulator path's: 8 int32 arrays per row of x and
// of w (top, low, need, list, pos, tail count, tail offset, recompute list),
// the span histogram and the plan's words; SL_MAX digits of x (rows padded to 128) and of w
// (rows padded to 128), K padded to 128; for K > 2^14 the 128-bit sums
// [M][N] carried between launches; the tails' k (SL_TAIL_CAP per row); the
// listed outputs' 128-bit sums (at most SL_ZFIX_MAX, and 2MN).
int64_t slice_rows_x(int64_t M) { return round_up(M, 128); }
int64_t slice_rows_w(int64_t N) { return round_up(N, 128); }
int64_t slice_stats_bytes(int64_t M, int64_t N) { return round_up(32 * (M + N) + 4 * (2 * SL_HIST + PL_WORDS), 256); }
int64_t slice_zfix_outputs(int64_t M, int64_t N) { return min(SL_ZFIX_MAX, 2 * M * N); }
int64_t slice_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t Kp = round_up(K, 2 * SL_KB);
  return slice_stats_bytes(M, N) + SL_MAX * (slice_rows_x(M) + slice_rows_w(N)) * Kp +
         (Kp / SL_KB > SL_FOLD ? 16 * M * N : 0) + 4 * SL_TAIL_CAP * (M + N) + 16 * slice_zfix_outputs(M, N);
}


std::atomic<int> g_path{DET_PATH_AUTO};
std::atomic<int> g_forced_slices{0};
// Pinned host buffer for the span histogram that DET_PATH_AUTO_HOST reads
// back, per calling thread, grown on demand and kept until the process ends:
// a copy into pinned memory is asynchronous, while one into pageable memory
// makes the host wait for it.  Every such call has waited for its copy
// before it returns, so the buffer is never replaced while a copy into it is
// in flight.
struct Pinned {
  int32_t* p = nullptr;
  size_t n = 0;
};
thread_local Pinned g_pin_hist;

int32_t* pinned(Pinned& b, size_t n) {
  if (b.n < n) {
    if (b.p != nullptr) (void)hipHostFree(b.p);
    b.p = nullptr;
    b.n = 0;
    void* q = nullptr;
    if (hipHostMalloc(&q, n * sizeof(int32_t), hipHostMallocDefault) != hipSuccess) return nullptr;
    b.p = static_cast<int32_t*>(q);
    b.n = n;
  }
  return b.p;
}

// wait for an event by polling it: the readbacks are short and each one
// holds up the launches that follow it
det_status poll_event(hipEvent_t ev, const char* what) {
  for (;;) {
    const hipError_t q = hipEventQuery(ev);
    if (q == hipSuccess) return DET_OK;
    if (q != hipErrorNotReady) return hip_check(q, what);
  }
}

// What the calling thread's last det_gemm call did, for det_last_gemm_plan.
// A path the host chose is kept here; a plan made on the device is copied,
// after its kernel, into one of four pinned slots per thread (a ring, so a
// copy never lands in a slot whose previous copy may still be in flight: the
// stream waits for that one first) and read when it is asked for.
struct PlanLog {
  int32_t* rec = nullptr;                 // pinned, 4 slots of PL_WORDS
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
  int dev[4] = {-1, -1, -1, -1};
  int next = 0;
  int last = -1;                          // slot of the last call's device plan; -1: the host's below
  det_path path = DET_PATH_ACCUMULATOR;
  int slices = 0;
  int64_t rows = 0, cols = 0;
};
thread_local PlanLog g_plan_log;

void record_plan(det_path p, int S, int64_t fx, int64_t fw) {
  PlanLog& l = g_plan_log;
  l.last = -1;
  l.path = p; l.slices = S; l.rows = fx; l.cols = fw;
}

// copy the device plan `plan` into the next slot, in stream order (not under
// graph capture: the record is then unknown)
det_status log_device_plan(const int32_t* plan, hipStream_t s) {
  PlanLog& l = g_plan_log;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  det_status st0 = hip_check(hipStreamIsCapturing(s, &cs), "capture status");
  if (st0 != DET_OK) return st0;
  if (cs != hipStreamCaptureStatusNone) {
    record_plan(DET_PATH_AUTO, -1, -1, -1);
    return DET_OK;
  }
  if (l.rec == nullptr) {
    void* q = nullptr;
    det_status st = hip_check(hipHostMalloc(&q, 4 * PL_WORDS * sizeof(int32_t), hipHostMallocDefault),
                              "pinned plan record");
    if (st != DET_OK) return st;
    l.rec = static_cast<int32_t*>(q);
  }
  int dev = -1;
  det_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (st != DET_OK) return st;
  const int i = l.next;
  l.next = (i + 1) & 3;
  if (l.ev[i] != nullptr && l.dev[i] != dev) {
    (void)hipEventSynchronize(l.ev[i]);             // another device's copy: let it land, then drop its event
    (void)hipEventDestroy(l.ev[i]);
    l.ev[i] = nullptr;
  }
  if (l.ev[i] == nullptr) {
    st = hip_check(hipEventCreateWithFlags(&l.ev[i], hipEventDisableTiming), "event create");
    if (st != DET_OK) return st;
    l.dev[i] = dev;
  } else {
    st = hip_check(hipStreamWaitEvent(s, l.ev[i], 0), "plan record order");
    if (st != DET_OK) return st;
  }
  st = hip_check(hipMemcpyAsync(l.rec + i * PL_WORDS, plan, PL_WORDS * sizeof(int32_t), hipMemcpyDeviceToHost, s),
                 "plan record copy");
  if (st == DET_OK) st = hip_check(hipEventRecord(l.ev[i], s), "event record");
  if (st == DET_OK) l.last = i;
  return st;
}

int choose_slices(det_dtype dt, int64_t M, int64_t N, int64_t K, const int32_t* hx, const int32_t* hw,
                  bool only_slices, int forced, int64_t& fx, int64_t& fw) {
  const double macs = static_cast<double>(M) * N * K;
  const double rate_acc = dt == DET_F32 ? RATE_ACC_F32 : RATE_ACC_BF16;
  double best = only_slices ? 1e300 : macs / rate_acc;
  int best_s = 0;
  for (int S = SL_MIN; S <= SL_MAX; ++S) {
    if (forced != 0 && S != forced) continue;
    int64_t cx = 0, cw = 0;
    for (int n = S + 1; n <= SL_MAX + 1; ++n) { cx += hx[n]; cw += hw[n]; }
    const double t = static_cast<double>(S) * S * macs / RATE_MMA +
                     (static_cast<double>(cx) * N * K + static_cast<double>(cw) * M * K) / rate_acc;
    if (t < best) { best = t; best_s = S; fx = cx; fw = cw; }
  }
  return best_s;
}

// tile shapes: 16-column blocks per wave, wave rows, LDS buffers
template <int S> struct SliceShape;
template <> struct SliceShape<2> { static constexpr int CB = 4, WR = 2, NBUF = 2; };
template <> struct SliceShape<3> { static constexpr int CB = 2, WR = 2, NBUF = 2; };
template <> struct SliceShape<4> { static constexpr int CB = 2, WR = 2, NBUF = 2; };
template <> struct SliceShape<5> { static constexpr int CB = 1, WR = 2, NBUF = 2; };
template <> struct SliceShape<6> { static constexpr int CB = 1, WR = 2, NBUF = 2; };
template <> struct SliceShape<7> { static constexpr int CB = 1, WR = 2, NBUF = 2; };

// the launches of one pass over K, in blocks of 2^14 k (SL_FOLD steps) so
// that each int32 sum stays below 2^31: `go(b)` launches block b
template <class Go>
det_status launch_mma_kblocks(const SliceMmaArgs& m, hipStream_t s, int marks, Go go) {
  const int64_t nblk = (m.Kb + SL_FOLD - 1) / SL_FOLD;
  for (int64_t ib = 0; ib < nblk; ++ib) {
    SliceMmaArgs b = m;
    b.kb0 = ib * SL_FOLD;
    b.kb1 = min(m.Kb, b.kb0 + SL_FOLD);
    b.epi = nblk == 1 ? EPI_ROUND : ib == 0 ? EPI_STORE : ib + 1 == nblk ? EPI_ADD_ROUND : EPI_ADD;
    det_status st = mark_event(g_ev_start, (marks & MARK_START) && ib == 0, s);
    if (st != DET_OK) return st;
    go(b);
    st = hip_check(hipGetLastError(), "slice mma launch");
    if (st == DET_OK) st = mark_event(g_ev_stop, (marks & MARK_STOP) && ib + 1 == nblk, s);
    if (st != DET_OK) return st;
  }
  return DET_OK;
}

template <int S, int CB>
det_status launch_mma_cb(SliceMmaArgs m, hipStream_t s, int marks) {
  using Sh = SliceShape<S>;
  constexpr int WR = Sh::WR, NBUF = Sh::NBUF;
  static_assert(SliceTile<S, CB, WR, NBUF>::LDS_BYTES <= 160 * 1024, "LDS");
  m.tiles_m = slice_rows_x(m.M) / (32 * WR);
  m.tiles_n = (m.N + 32 * CB - 1) / (32 * CB);
  const int64_t blocks = m.tiles_m * m.tiles_n;
  if (blocks > 0x7FFFFFFF) return fail(DET_EINVAL, "too many output tiles");
  const dim3 grid(static_cast<unsigned>(blocks)), block(128 * WR);
  return launch_mma_kblocks(m, s, marks, [&](const SliceMmaArgs& b) {
    hipLaunchKernelGGL((k_slice_mma<S, CB, WR, NBUF>), grid, block, 0, s, b);
  });
}

// A product with at most 1024 tiles of the regular shape leaves slots of the
// 256 CUs (two workgroups each) idle for much of the kernel: it takes tiles
// half as wide, twice as many (measured: bf16 512^3 58.7 -> 51.2 us, 1024^3
// 78 -> 70 us, 2048^3 203 -> 197 us; the 8192 x 4096 x 4096 shape is
// faster with the regular tiles, 1.61 against 1.65 ms).
template <int S>
det_status launch_mma(SliceMmaArgs m, hipStream_t s, int marks) {
  constexpr int CB = SliceShape<S>::CB, WR = SliceShape<S>::WR;
  const int64_t tiles = slice_rows_x(m.M) / (32 * WR) * ((m.N + 32 * CB - 1) / (32 * CB));
  if constexpr (CB > 1) {
    if (tiles <= 1024) return launch_mma_cb<S, CB / 2>(m, s, marks);
  }
  return launch_mma_cb<S, CB>(m, s, marks);
}

// Whether S = 2 .. 6 go in one launch of k_slice_mma_small: every S takes
// the narrow tiles of launch_mma (at most 1024 tiles of 64 x 64), and the
// product is small enough that the launches saved outweigh the merged
// kernel's lower occupancy (its registers are those of S = 6: two
// workgroups per CU where S = 4 alone fits three).  Measured on bf16 N(0,1):
// 1024^3 84 -> 72 us per call, 512^3 61 -> 52 us; 2048^3 (1024 tiles)
// 192 -> 196 us, so it keeps a launch per S.
bool mma_small(int64_t M, int64_t N) { return slice_rows_x(M) / 64 * ((N + 63) / 64) <= 512; }

det_status launch_mma_small(SliceMmaArgs m, hipStream_t s, int marks) {
  static_assert(SL_MIN == 2 && SL_MAX == 7, "k_slice_mma_small holds S = 2 .. 6");
  static_assert(SliceShape<2>::CB == 2 * SMALL_CB[2] && SliceShape<3>::CB == 2 * SMALL_CB[3] &&
                SliceShape<4>::CB == 2 * SMALL_CB[4] && SliceShape<5>::CB == SMALL_CB[5] &&
                SliceShape<6>::CB == SMALL_CB[6], "the narrow shapes of launch_mma");
  const int64_t blocks = slice_rows_x(m.M) / 64 * ((m.N + 31) / 32);     // the largest count: 32 columns
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  return launch_mma_kblocks(m, s, marks, [&](const SliceMmaArgs& b) {
    hipLaunchKernelGGL(k_slice_mma_small, grid, block, 0, s, b);
  });
}

// one operand's span-check arguments and its block count
template <int DT>
SliceStatArgs stat_args(const void* p, int64_t R, int64_t K, int64_t s_r, int64_t s_k, int32_t* top, int32_t* low,
                        int64_t& blocks) {
  SliceStatArgs a{p, R, K, s_r, s_k, top, low, false, false};
  const int64_t esz = DT == DET_F32 ? 4 : 2;
  const bool aligned = (reinterpret_cast<uintptr_t>(p) % 16) == 0;
  a.vec = s_k == 1 ? aligned && (s_r * esz) % 16 == 0 : s_r == 1 && aligned && (s_k * esz) % 16 == 0;
  a.direct = K <= (s_k == 1 ? STAT_KR : 256);
  blocks = s_k == 1 ? (R * ((K + STAT_KR - 1) / STAT_KR) + 3) / 4
         : a.vec    ? (R + 63) / 64 * ((K + 255) / 256)
                    : (R * ((K + 255) / 256) + 255) / 256;
  return a;
}

// x's and w's span checks: one launch when both have the same layout.  The
// tops and lows of x then w are adjacent (topx, lowx hold M + N entries);
// they need initial values only where several waves share a row.
template <int DT>
det_status slice_stats(const GemmArgs& g, int32_t* topx, int32_t* lowx, int32_t* topw, int32_t* loww,
                       int32_t* hist, hipStream_t s) {
  int64_t bx, bw;
  const SliceStatArgs ax = stat_args<DT>(g.x, g.M, g.K, g.x_sm, g.x_sk, topx, lowx, bx);
  const SliceStatArgs aw = stat_args<DT>(g.w, g.N, g.K, g.w_sn, g.w_sk, topw, loww, bw);
  if (!ax.direct || !aw.direct) {
    hipLaunchKernelGGL(k_slice_init, dim3(grid_for(g.M + g.N, 256, 1024)), dim3(256), 0, s, topx, lowx, g.M + g.N);
    det_status st = hip_check(hipGetLastError(), "slice init launch");
    if (st != DET_OK) return st;
  }
  bool first = true;
  auto launch = [&](const SliceStatArgs& a0, int64_t b0, const SliceStatArgs& a1, int64_t b1, bool kmaj) {
    SliceStatPair p{{a0, a1}, b0, first ? hist : nullptr};
    first = false;
    const dim3 grid(static_cast<unsigned>(b0 + b1));
    if (kmaj) hipLaunchKernelGGL((k_slice_stats<DT, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_slice_stats<DT, false>), grid, dim3(256), 0, s, p);
  };
  const bool kx = g.x_sk == 1, kw = g.w_sk == 1;
  if (kx == kw) {
    launch(ax, bx, aw, bw, kx);
  } else {
    launch(ax, bx, ax, 0, kx);
    launch(aw, bw, aw, 0, kw);
  }
  return hip_check(hipGetLastError(), "slice stats launch");
}

// one operand's digit-making arguments; `trans`: the LDS-transposing form
template <int DT>
SliceMakeArgs make_args(const void* p, int64_t R, int64_t K, int64_t s_r, int64_t s_k, const int32_t* top,
                        int8_t* out, int64_t rows_padded, int S, bool& trans, int64_t& blocks) {
  const int64_t esz = DT == DET_F32 ? 4 : 2;
  SliceMakeArgs a{};
  a.p = p; a.R = R; a.K = K; a.s_r = s_r; a.s_k = s_k; a.top = top; a.out = out;
  a.Rb = rows_padded / 16; a.Kb = round_up(K, 2 * SL_KB) / SL_KB;
  a.S = S;
  trans = s_r == 1 && s_k > 1;            // a transposed view: through LDS (Rb is a multiple of 8)
  // 16-byte loads along k (K-major) or along the rows (transposed)
  a.vec = (reinterpret_cast<uintptr_t>(p) % 16) == 0 &&
          (trans ? (s_k * esz) % 16 == 0 : s_k == 1 && (s_r * esz) % 16 == 0);
  blocks = trans ? a.Rb / 4 * a.Kb : grid_for(a.Rb * a.Kb * 64, 256, 8192);
  return a;
}

// x's and w's digits: one launch when both take the same form
template <int DT>
det_status slice_make(const GemmArgs& g, const int32_t* topx, const int32_t* topw, int8_t* xs, int8_t* wsl,
                      const int32_t* plan, hipStream_t s) {
  bool tx, tw;
  int64_t bx, bw;
  const SliceMakeArgs ax = make_args<DT>(g.x, g.M, g.K, g.x_sm, g.x_sk, topx, xs, slice_rows_x(g.M), 0, tx, bx);
  const SliceMakeArgs aw = make_args<DT>(g.w, g.N, g.K, g.w_sn, g.w_sk, topw, wsl, slice_rows_w(g.N), 0, tw, bw);
  auto launch = [&](const SliceMakeArgs& a0, int64_t b0, const SliceMakeArgs& a1, int64_t b1, bool trans) {
    SliceMakePair p{{a0, a1}, b0, b1, plan};
    const dim3 grid(static_cast<unsigned>(b0 + b1));
    if (trans) hipLaunchKernelGGL((k_slice_make_t<DT>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((k_slice_make<DT>), grid, dim3(256), 0, s, p);
  };
  if (tx == tw) {
    launch(ax, bx, aw, bw, tx);
  } else {
    launch(ax, bx, ax, 0, tx);
    launch(aw, bw, aw, 0, tw);
  }
  return hip_check(hipGetLastError(), "slice make launch");
}

template <int DT>
det_status launch_gemm8(GemmArgs a, void* ws, hipStream_t s, int marks);

// The accumulator path on a subset whose size the device decided: the
// *count rows `rows` of x (and all of w), or the *count rows `cols` of w
// (and all of x), overwriting those outputs of y; nothing when *count is 0.
// One launch: the kernel reads the raw operands through the maps (no
// pre-decode launch, no workspace), which costs a skipped recompute one
// dispatch instead of three.
template <int DT>
det_status recompute(GemmArgs a, const int32_t* rows, const int32_t* cols, const int32_t* count, hipStream_t s) {
  GemmArgs b = a;
  b.xmap = rows; b.wmap = cols;
  b.gate = count;
  if (rows != nullptr) b.mcount = count;
  else b.ncount = count;
  return launch_gemm8<DT>(b, nullptr, s, 0);
}

// det_gemm with the room for both paths in `ws`: span statistics, then the
// plan, made on the device (by k_slice_need's last workgroup) so that the
// host never waits: the
// kernels of every path the plan may pick are enqueued, each reading the
// plan and doing nothing unless it is the one picked.  With `host_choice`
// (DET_PATH_AUTO_HOST) the host instead waits for the histogram, picks, and
// enqueues only that path.  Rows whose span needs more than S digits
// ("listed") keep their matrix-core sums; their tails' products are added
// one by one (k_slice_fix), or, for rows with more than SL_TAIL_CAP tails or
// more listed outputs than the sums' room, the accumulator path recomputes
// them (a grid that takes the device-counted rows in turn).
template <int DT>
det_status launch_sliced(GemmArgs a, char* ws, bool only_slices, int forced, bool host_choice, hipStream_t s) {
  const int64_t M = a.M, N = a.N, K = a.K;
  char* const sl = ws + workspace_bytes(1, M, N, K);
  int32_t* q = reinterpret_cast<int32_t*>(sl);
  auto take = [&](int64_t n) { int32_t* r = q; q += n; return r; };
  int32_t* const topx = take(M); int32_t* const topw = take(N);      // top, then low: contiguous for init
  int32_t* const lowx = take(M); int32_t* const loww = take(N);
  int32_t* const needx = take(M); take(N);                           // need of x, then of w
  int32_t* const listx = take(M); int32_t* const listw = take(N);
  int32_t* const posx = take(M); int32_t* const posw = take(N);
  int32_t* const cntx = take(M); int32_t* const cntw = take(N);
  int32_t* const offx = take(M); int32_t* const offw = take(N);
  int32_t* const ovlx = take(M); int32_t* const ovlw = take(N);
  int32_t* const hist = take(2 * SL_HIST);
  int32_t* const plan = take(PL_WORDS);
  const int64_t Kp = round_up(K, 2 * SL_KB);
  char* r8 = sl + slice_stats_bytes(M, N);
  int8_t* const xs = reinterpret_cast<int8_t*>(r8);
  int8_t* const wsl = xs + SL_MAX * slice_rows_x(M) * Kp;
  r8 += SL_MAX * (slice_rows_x(M) + slice_rows_w(N)) * Kp;
  int64_t* const zcarry = reinterpret_cast<int64_t*>(r8);
  if (Kp / SL_KB > SL_FOLD) r8 += 16 * M * N;
  int32_t* const tkx = reinterpret_cast<int32_t*>(r8);
  int32_t* const tkw = tkx + SL_TAIL_CAP * M;
  r8 += 4 * SL_TAIL_CAP * (M + N);
  int64_t* const zfix = reinterpret_cast<int64_t*>(r8);

  det_status st = slice_stats<DT>(a, topx, lowx, topw, loww, hist, s);
  if (st != DET_OK) return st;
  int mode = only_slices ? forced : 0;              // > 0: S fixed here
  PlanArgs pa{};
  pa.hist = hist; pa.plan = plan;
  pa.M = M; pa.N = N; pa.K = K; pa.zfix = slice_zfix_outputs(M, N);
  pa.rate_acc = DT == DET_F32 ? RATE_ACC_F32 : RATE_ACC_BF16;
  pa.mode = mode; pa.only = only_slices; pa.forced = forced;
  // x's and w's tops, lows and needs are adjacent: one pass over M + N rows,
  // whose last workgroup makes the plan (unless the host picks the path)
  hipLaunchKernelGGL(k_slice_need, dim3(grid_for(M + N, 256, 256)), dim3(256), 0, s, topx, lowx, M + N, M, needx,
                     hist, cntx, pa, host_choice ? 0 : 1);
  st = hip_check(hipGetLastError(), "slice need launch");
  if (st != DET_OK) return st;

  if (host_choice) {
    int32_t* const h = pinned(g_pin_hist, 2 * SL_HIST);
    if (h == nullptr) return fail(DET_EHIP, "pinned host buffer for the span histogram");
    hipEvent_t ready = nullptr;
    st = hip_check(hipMemcpyAsync(h, hist, 2 * SL_HIST * sizeof(int32_t), hipMemcpyDeviceToHost, s),
                   "span histogram copy");
    if (st == DET_OK) st = hip_check(hipEventCreateWithFlags(&ready, hipEventDisableTiming), "event create");
    if (st == DET_OK) st = hip_check(hipEventRecord(ready, s), "event record");
    if (st == DET_OK) st = poll_event(ready, "span histogram wait");
    if (ready != nullptr) (void)hipEventDestroy(ready);
    if (st != DET_OK) return st;
    int64_t fx = 0, fw = 0;
    mode = choose_slices(static_cast<det_dtype>(DT), M, N, K, h, h + SL_HIST, only_slices, forced, fx, fw);
    if (mode == 0) {
      record_plan(DET_PATH_ACCUMULATOR, 0, 0, 0);
      return launch_gemm8<DT>(a, ws, s);
    }
  }
  if (host_choice) {
    pa.mode = mode;
    hipLaunchKernelGGL(k_slice_plan, dim3(1), dim3(64), 0, s, pa);
    st = hip_check(hipGetLastError(), "plan launch");
  }
  if (st == DET_OK) st = log_device_plan(plan, s);
  if (st != DET_OK) return st;

  // the accumulator path, if the plan may pick it (the kernel timing
  // events then wrap its launches, picked or not)
  const bool acc_alt = mode == 0 && !only_slices;
  if (acc_alt) {
    GemmArgs b = a;
    b.gate = plan + PL_ACC;
    st = launch_gemm8<DT>(b, ws, s, MARK_BOTH);
    if (st != DET_OK) return st;
  }
  hipLaunchKernelGGL(k_slice_list, dim3(2), dim3(1024), 0, s, needx, M, N, plan, listx, posx);
  st = hip_check(hipGetLastError(), "slice list launch");
  if (st != DET_OK) return st;
  // tails per listed row (when the plan keeps tails)
  {
    const int64_t nkr = (K + 1023) / 1024;
    TailPair tp{};
    TailArgs& t = tp.op[0];
    t.p = a.x; t.K = K; t.s_r = a.x_sm; t.s_k = a.x_sk; t.list = listx; t.top = topx; t.plan = plan; t.side = 0;
    t.cnt = cntx; t.tk = tkx;
    TailArgs& u = tp.op[1];
    u = t;
    u.p = a.w; u.s_r = a.w_sn; u.s_k = a.w_sk; u.list = listw; u.top = topw; u.side = 1;
    u.cnt = cntw; u.tk = tkw;
    tp.nb0 = grid_for(M * nkr * 64, 256, 1024);
    const int64_t nb1 = grid_for(N * nkr * 64, 256, 1024);
    hipLaunchKernelGGL((k_tail_scan<DT>), dim3(static_cast<unsigned>(tp.nb0 + nb1)), dim3(256), 0, s, tp);
    st = hip_check(hipGetLastError(), "tail count launch");
    if (st != DET_OK) return st;
  }
  st = slice_make<DT>(a, topx, topw, xs, wsl, plan, s);
  if (st != DET_OK) return st;
  SliceMmaArgs m{};
  m.xs = xs; m.ws = wsl;
  m.Kb = Kp / SL_KB;
  m.M = M; m.N = N;
  m.topx = topx; m.topw = topw;
  m.y = a.y; m.y_sm = a.y_sm; m.y_sn = a.y_sn;
  m.z = zcarry;
  m.posx = posx; m.posw = posw;
  m.zr = zfix; m.zc = nullptr;                 // behind the listed rows' sums: set on the device
  m.plan = plan;
  // every S the plan may pick; without the accumulator's launches the
  // timing interval runs from the first to the last
  const int s_lo = mode > 0 ? mode : (forced != 0 ? forced : SL_MIN);
  const int s_hi = mode > 0 ? mode : (forced != 0 ? forced : SL_MAX);
  int s_next = s_lo;
  if (s_lo == SL_MIN && s_hi == SL_MAX && mma_small(M, N)) {     // S = 2 .. 6 in one launch
    st = launch_mma_small(m, s, acc_alt ? 0 : MARK_START);
    s_next = SL_MAX;
  }
  for (int S = s_next; S <= s_hi && st == DET_OK; ++S) {
    const int marks = acc_alt ? 0 : (S == s_lo ? MARK_START : 0) | (S == s_hi ? MARK_STOP : 0);
    switch (S) {
      case 2: st = launch_mma<2>(m, s, marks); break;
      case 3: st = launch_mma<3>(m, s, marks); break;
      case 4: st = launch_mma<4>(m, s, marks); break;
      case 5: st = launch_mma<5>(m, s, marks); break;
      case 6: st = launch_mma<6>(m, s, marks); break;
      default: st = launch_mma<7>(m, s, marks); break;
    }
  }
  if (st != DET_OK) return st;
  // which listed rows go to the accumulator path, and the tails of the others
  hipLaunchKernelGGL(k_tail_plan, dim3(2), dim3(1024), 0, s, plan, M, cntx, listx, offx, ovlx);
  SliceFixArgs f{};
  f.x = a.x; f.x_sm = a.x_sm; f.x_sk = a.x_sk;
  f.w = a.w; f.w_sn = a.w_sn; f.w_sk = a.w_sk;
  f.M = M; f.N = N;
  f.topx = topx; f.topw = topw; f.listx = listx; f.listw = listw; f.posx = posx; f.posw = posw;
  f.cntx = cntx; f.cntw = cntw; f.offx = offx; f.offw = offw; f.tkx = tkx; f.tkw = tkw;
  f.zr = m.zr; f.zc = m.zc;
  f.y = a.y; f.y_sm = a.y_sm; f.y_sn = a.y_sn;
  f.plan = plan;
  hipLaunchKernelGGL((k_slice_fix<DT>), dim3(grid_for(slice_zfix_outputs(M, N), 256, 4096)), dim3(256), 0, s, f);
  st = hip_check(hipGetLastError(), "tail launch");
  // rows and columns the accumulator path recomputes
  if (st == DET_OK) st = recompute<DT>(a, ovlx, nullptr, plan + PL_OX, s);
  if (st == DET_OK) st = recompute<DT>(a, nullptr, ovlw, plan + PL_OW, s);
  return st;
}

det_status launch_gemm(det_dtype dt, int out_mode, GemmArgs a, void* ws, hipStream_t s) {
  if (out_mode == 0) return dt == DET_F32 ? launch_partial<DET_F32>(a, ws, s) : launch_partial<DET_BF16>(a, ws, s);
  return dt == DET_F32 ? launch_gemm8<DET_F32>(a, ws, s) : launch_gemm8<DET_BF16>(a, ws, s);
}

// ---------------------------------------------------------------- static scratch
//
// det_gemm_noalloc keeps its workspace (w and x decoded, and the digits carried
// between K blocks) in this file-scope array instead of memory the caller
// brings in: every GPU the library runs on holds one copy until the process
// ends, and every det_gemm_noalloc call on that GPU shares it.  In host code
// `scratch` names a host-side stand-in, not device memory: the kernels get the
// array's device address, looked up once per device.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

// the current device's copy of `scratch` (its address is fixed for the life of
// the process), looked up with that device current on first use
det_status scratch_for_current_device(void** out) {
  int dev = -1;
  det_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (st != DET_OK) return st;
  if (dev < 0 || dev >= MAX_DEVICES) return fail(DET_EINVAL, "device %d is beyond the %d supported", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    st = hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "scratch symbol address");
    if (st != DET_OK) return st;
    if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u)) return fail(DET_EHIP, "scratch address %p", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DET_OK;
}

// the current device's copy of g_dev_status, looked up once per device
std::mutex g_status_mu;
void* g_status_ptr[MAX_DEVICES];

det_status status_words(void** out) {
  int dev = -1;
  det_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (st != DET_OK) return st;
  if (dev < 0 || dev >= MAX_DEVICES) return fail(DET_EINVAL, "device %d is beyond the %d supported", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_status_mu);
  if (g_status_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    st = hip_check(hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_dev_status)), "status symbol address");
    if (st != DET_OK) return st;
    if (ptr == nullptr) return fail(DET_EHIP, "status word address is null");
    g_status_ptr[dev] = ptr;
  }
  *out = g_status_ptr[dev];
  return DET_OK;
}

__global__ __launch_bounds__(64) void k_status_clear(int32_t* words) {
  if (threadIdx.x < 4) words[threadIdx.x] = 0;
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
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (out_mode == 1 && ws != nullptr && M > 0 && N > 0 && K > 0) {
    const int path = g_path.load();
    const bool room = ws_bytes >= static_cast<size_t>(workspace_bytes(1, M, N, K) + slice_bytes(M, N, K));
    if (path == DET_PATH_SLICES && !room)
      return fail(DET_EINVAL, "the matrix-core path needs a workspace of %lld bytes",
                  (long long)(workspace_bytes(1, M, N, K) + slice_bytes(M, N, K)));
    const bool big = static_cast<double>(M) * N * K >= SLICE_MIN_MACS;
    const bool autop = path == DET_PATH_AUTO || path == DET_PATH_AUTO_HOST;
    if (room && (path == DET_PATH_SLICES || (autop && big))) {
      const bool only = path == DET_PATH_SLICES, host = path == DET_PATH_AUTO_HOST;
      const int forced = only ? g_forced_slices.load() : 0;
      char* const w8 = static_cast<char*>(ws);
      return dt == DET_F32 ? launch_sliced<DET_F32>(a, w8, only, forced, host, s)
                           : launch_sliced<DET_BF16>(a, w8, only, forced, host, s);
    }
  }
  if (out_mode == 1) record_plan(DET_PATH_ACCUMULATOR, 0, 0, 0);
  return launch_gemm(dt, out_mode, a, ws, s);
}

}  // namespace

int64_t det_gemm_workspace_bytes(det_dtype dt, int partial, int64_t M, int64_t N, int64_t K) {
  (void)dt;
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (partial) return workspace_bytes(0, M, N, K);
  return workspace_bytes(1, M, N, K) + slice_bytes(M, N, K);
}

det_status det_set_gemm_path(det_path path, int slices) {
  if (path != DET_PATH_AUTO && path != DET_PATH_ACCUMULATOR && path != DET_PATH_SLICES &&
      path != DET_PATH_AUTO_HOST)
    return fail(DET_EINVAL, "unknown path %d", static_cast<int>(path));
  if (slices != 0 && (slices < SL_MIN || slices > SL_MAX))
    return fail(DET_EINVAL, "slices must be 0 or %d..%d (got %d)", SL_MIN, SL_MAX, slices);
  g_forced_slices.store(slices);
  g_path.store(static_cast<int>(path));
  return DET_OK;
}

void det_get_gemm_path(det_path* path, int* slices) {
  if (path) *path = static_cast<det_path>(g_path.load());
  if (slices) *slices = g_forced_slices.load();
}

void det_last_gemm_plan(int* path, int* slices, int64_t* fallback_rows, int64_t* fallback_cols) {
  PlanLog& l = g_plan_log;
  if (l.last >= 0) {                              // made on the device: wait for its copy
    const int32_t* r = l.rec + l.last * PL_WORDS;
    if (hipEventSynchronize(l.ev[l.last]) == hipSuccess) {
      l.path = r[PL_S] > 0 ? DET_PATH_SLICES : DET_PATH_ACCUMULATOR;
      l.slices = r[PL_S];
      l.rows = r[PL_S] > 0 ? r[PL_FX] : 0;
      l.cols = r[PL_S] > 0 ? r[PL_FW] : 0;
    } else {
      l.path = DET_PATH_AUTO; l.slices = -1; l.rows = l.cols = -1;    // unknown
    }
    l.last = -1;
  }
  if (path) *path = static_cast<int>(l.path);
  if (slices) *slices = l.slices;
  if (fallback_rows) *fallback_rows = l.rows;
  if (fallback_cols) *fallback_cols = l.cols;
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

det_status det_device_status(void* stream, int clear, int* flags) {
  if (flags != nullptr) *flags = 0;
  void* p = nullptr;
  det_status st = status_words(&p);
  if (st != DET_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t h[4] = {0, 0, 0, 0};
  st = hip_check(hipMemcpyAsync(h, p, sizeof h, hipMemcpyDeviceToHost, s), "status copy");
  if (st == DET_OK && clear) {
    hipLaunchKernelGGL(k_status_clear, dim3(1), dim3(64), 0, s, static_cast<int32_t*>(p));
    st = hip_check(hipGetLastError(), "status clear launch");
  }
  const det_status sync = hip_check(hipStreamSynchronize(s), "status wait");
  if (st == DET_OK) st = sync;
  if (st != DET_OK) return st;
  const int f = (h[0] != 0 ? 1 : 0) | (h[1] != 0 ? 2 : 0);
  if (flags != nullptr) *flags = f;
  if (f & 1) return fail(DET_ENONFINITE, "an operand held Inf or NaN");
  if (f & 2) return fail(DET_ERANGE, "a digit lay outside +-2^62");
  return DET_OK;
}

int32_t* det_device_status_word(void) {
  void* p = nullptr;
  return status_words(&p) == DET_OK ? static_cast<int32_t*>(p) : nullptr;
}

void det_set_kernel_events(void* start, void* stop) {
  g_ev_start = static_cast<hipEvent_t>(start);
  g_ev_stop = static_cast<hipEvent_t>(stop);
}

size_t det_gemm_noalloc_max_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

det_status det_gemm_noalloc(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk, const void* w,
                            int64_t w_sn, int64_t w_sk, int64_t M, int64_t N, int64_t K, float* y,
                            int64_t y_sm, int64_t y_sn, void* stream) {
  det_status st = check_operands(dt, x, x_sm, x_sk, w, w_sn, w_sk, M, N, K);
  if (st != DET_OK) return st;
  if (M > 0 && N > 0 && y == nullptr) return fail(DET_EINVAL, "null output");
  if (y_sm < 0 || y_sn < 0) return fail(DET_EINVAL, "negative output stride");
  if (reinterpret_cast<uintptr_t>(y) & 3u) return fail(DET_EINVAL, "output must be 4-byte aligned");
  // the accumulator path's workspace: decoded w, one K block of decoded x,
  // and for K > 2^15 the digits carried between blocks
  const double need = static_cast<double>(round_up(N, V_BN)) * round_up(K, V_KC) * 8 +
                      static_cast<double>(round_up(M, TILE_ROWS)) * round_up(min(K, K_BLOCK), V_KC) * 8 +
                      (K > K_BLOCK ? 144.0 * static_cast<double>(M) * static_cast<double>(N) : 0.0);
  if (need > static_cast<double>(NOALLOC_SCRATCH_BYTES))
    return fail(DET_EINVAL, "det_gemm_noalloc: M=%lld N=%lld K=%lld needs %.0f bytes of scratch, more than its %zu",
                (long long)M, (long long)N, (long long)K, need, NOALLOC_SCRATCH_BYTES);
  if (M == 0 || N == 0) return DET_OK;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != DET_OK) return st;
  GemmArgs a{};
  a.x = x; a.x_sm = x_sm; a.x_sk = x_sk;
  a.w = w; a.w_sn = w_sn; a.w_sk = w_sk;
  a.M = M; a.N = N; a.K = K;
  a.y = y; a.y_sm = y_sm; a.y_sn = y_sn;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dt == DET_F32 ? launch_gemm8<DET_F32>(a, ws, s) : launch_gemm8<DET_BF16>(a, ws, s);
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
  // `out` may be one of the parts (the same pointer); any other overlap with
  // a part is rejected.  Parts equal to `out` go into the first launch, which
  // reads every element of its parts before it writes that element of `out`:
  // later launches would read `out` after it holds the running sum.
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), o1 = o0 + static_cast<uintptr_t>(n) * 8u;
  int aliased = 0;
  for (int p = 0; p < nparts; ++p) {
    const uintptr_t p0 = reinterpret_cast<uintptr_t>(parts[p]), p1 = p0 + static_cast<uintptr_t>(n) * 8u;
    if (p0 == o0) ++aliased;
    else if (p0 < o1 && o0 < p1) return fail(DET_EINVAL, "part %d overlaps out without being equal to it", p);
  }
  if (aliased > COMBINE_MAX)
    return fail(DET_EINVAL, "%d parts are equal to out; at most %d may be", aliased, COMBINE_MAX);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // more than COMBINE_MAX parts: fold them in groups, carrying the running sum
  // in `out` (integer addition: any grouping gives the same digits)
  int next_alias = 0, next_other = 0, done = 0;
  auto take = [&]() -> const int64_t* {
    while (next_alias < nparts && parts[next_alias] != out) ++next_alias;
    if (next_alias < nparts) return parts[next_alias++];
    while (parts[next_other] == out) ++next_other;
    return parts[next_other++];
  };
  while (done < nparts) {
    CombineArgs a{};
    a.out = out;
    a.n = n;
    if (done > 0) a.parts[a.nparts++] = out;
    while (a.nparts < COMBINE_MAX && done < nparts) {
      a.parts[a.nparts++] = take();
      ++done;
    }
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

det_status det_dot_partial(det_dtype dt, const void* a, int64_t inc_a, const void* b, int64_t inc_b, int64_t n,
                           int64_t* acc, int accumulate, void* stream) {
  return dot_common(DOT_PLAIN, dt, a, inc_a, b, inc_b, n, acc, accumulate, stream);
}

det_status det_sqdiff_partial(det_dtype dt, const void* a, int64_t inc_a, const void* b, int64_t inc_b,
                              int64_t n, int64_t* acc, int accumulate, void* stream) {
  return dot_common(b == nullptr ? DOT_SQUARE : DOT_SQDIFF, dt, a, inc_a, b, inc_b, n, acc, accumulate, stream);
}

det_status det_mse_grad(det_dtype dt, const void* y, const void* t, int64_t n, float c, const float* g, void* dy,
                        void* dt_out, void* stream) {
  if (dt != DET_F32 && dt != DET_BF16) return fail(DET_EDTYPE, "unknown dtype %d", static_cast<int>(dt));
  if (n < 0) return fail(DET_EINVAL, "negative count");
  if (n == 0 || (dy == nullptr && dt_out == nullptr)) return DET_OK;
  if (y == nullptr || g == nullptr) return fail(DET_EINVAL, "null pointer");
  const uintptr_t align = dt == DET_F32 ? 3u : 1u;
  if ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(t) | reinterpret_cast<uintptr_t>(dy) |
       reinterpret_cast<uintptr_t>(dt_out)) & align)
    return fail(DET_EINVAL, "operands must be aligned to their element size");
  if (reinterpret_cast<uintptr_t>(g) & 3u) return fail(DET_EINVAL, "g must be 4-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool vec = ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(t) | reinterpret_cast<uintptr_t>(dy) |
                     reinterpret_cast<uintptr_t>(dt_out)) & 15u) == 0;
  const dim3 grid(grid_for(vec ? (n + 7) / 8 : n, 256, 8192));
  if (dt == DET_F32) {
    if (vec) hipLaunchKernelGGL((k_mse_grad<DET_F32, true>), grid, dim3(256), 0, s, y, t, n, c, g, dy, dt_out);
    else hipLaunchKernelGGL((k_mse_grad<DET_F32, false>), grid, dim3(256), 0, s, y, t, n, c, g, dy, dt_out);
  } else {
    if (vec) hipLaunchKernelGGL((k_mse_grad<DET_BF16, true>), grid, dim3(256), 0, s, y, t, n, c, g, dy, dt_out);
    else hipLaunchKernelGGL((k_mse_grad<DET_BF16, false>), grid, dim3(256), 0, s, y, t, n, c, g, dy, dt_out);
  }
  return hip_check(hipGetLastError(), "mse gradient launch");
}

det_status det_round_f32_to_bf16(const float* in, uint16_t* out, int64_t n, void* stream) {
  if (n < 0) return fail(DET_EINVAL, "negative count");
  if (n == 0) return DET_OK;
  if (in == nullptr || out == nullptr) return fail(DET_EINVAL, "null pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint32_t* const b = reinterpret_cast<const uint32_t*>(in);
  int64_t done = 0;
  if (((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15u) == 0u && n >= 8) {
    hipLaunchKernelGGL(k_round_bf16<true>, dim3(static_cast<unsigned>((n / 8 + 255) / 256)), dim3(256), 0, s, b,
                       out, n);
    done = n / 8 * 8;
  }
  if (done < n)
    hipLaunchKernelGGL(k_round_bf16<false>, dim3(static_cast<unsigned>((n - done + 255) / 256)), dim3(256), 0, s,
                       b + done, out + done, n - done);
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
