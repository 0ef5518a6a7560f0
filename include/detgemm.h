/*
 * detgemm.h -- C ABI of the exact long-accumulator GEMM for AMD MI355X (gfx950).
 *
 * The operation is the one the det-train page defines ("Method" section):
 *
 *     y[m, n] = sum_k x[m, k] * w[n, k]
 *
 * where every product is exact, each product's base-2^32 limbs are added with
 * the product's sign into a per-output Kulisch long accumulator of signed
 * int64 digits, and the exact sum is rounded once to fp32.  Because the digit
 * sums are plain integer additions, the bits of every result are independent
 * of tiling, of how K is split, of the order in which partial accumulators
 * are added, and of repetition.  The interface follows the page's "Usage"
 * section (det_gemm, det_gemm_partial, det_combine, det_finalize); its limits
 * follow "Requirements and limits" (K <= 2^19 per call, bf16 and f32 inputs).
 *
 * Accumulator layout (the page states none; this is the library's reading):
 *   - DET_NUM_DIGITS = 18 signed int64 digits per output, digit j weighs
 *     2^(32*j - 298).  Digit 0 weighs 2^-298, the smallest nonzero product of
 *     two fp32 numbers; 18*32 = 576 bits hold every product (< 2^256) with
 *     headroom for 2^19 of them.
 *   - Digits are RAW sums: digit j is the sum over products of
 *     sign(p) * (bits [32j, 32j+32) of |p| * 2^298).  No carries are taken
 *     before rounding, so the digit arrays of K-slices add up, digit for
 *     digit, to the digit array of the whole K range.
 *   - An accumulator array is int64 [rows][cols][18], row-major, digit 0
 *     first, contiguous.
 *
 * Rounding (det_gemm, det_finalize): IEEE 754 binary32 round-to-nearest,
 * ties to even, gradual underflow, overflow to +-inf.  An exact zero gives
 * +0.0; a nonzero sum that rounds to zero keeps its sign (-0.0).
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no device memory (the _ws variants use memory the caller
 *     passes in); what it keeps on each GPU it runs on are two static device
 *     arrays, det_gemm_noalloc's workspace and the 16-byte status word of
 *     det_device_status, held until the process ends.  Host-side state, per
 *     calling thread and kept until the process ends: a 96-byte pinned
 *     buffer for the span histogram that DET_PATH_AUTO_HOST reads back, and
 *     four 32-byte pinned records with their events for det_last_gemm_plan.
 *   - Strides are in elements, must be >= 0, and may describe transposed or
 *     sliced views (e.g. x[:, a:b] or x^T).  Operand elements must be
 *     naturally aligned (4 bytes for f32, 2 for bf16).
 *   - The calling thread's current HIP device must be the device that holds
 *     the pointers and owns `stream` (the Python layer makes it current).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously and stream-ordered; no call waits for the device except
 *     the ones that say so: det_gemm_ws on the opt-in DET_PATH_AUTO_HOST,
 *     det_last_gemm_plan, det_device_status.  So every other call can be
 *     captured into a HIP graph.
 *   - Argument errors are reported before anything is enqueued; on error
 *     nothing is written.  det_last_error() returns a message for the calling
 *     thread's most recent failure.
 *   - Inputs must be finite (the page's limits name bf16 and f32 inputs and
 *     no others; the digits cannot hold Inf or NaN).  Because calls are
 *     asynchronous, an Inf or NaN operand is not an argument error: the
 *     kernels that read the operands note it in the device status (see
 *     det_device_status), which then reports DET_ENONFINITE, and the call's
 *     results are unspecified; every access stays in bounds all the same.
 *     Callers that want the check before any result is written run
 *     det_check_finite first.
 */
#ifndef DETGEMM_H
#define DETGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DET_NUM_DIGITS 18
#define DET_LSB_EXPONENT (-298)
#define DET_K_MAX ((int64_t)1 << 19)

typedef enum {
  DET_OK = 0,
  DET_EINVAL = 1,      /* bad pointer, size, stride or count */
  DET_EKLIMIT = 2,     /* K > 2^19 */
  DET_EDTYPE = 3,      /* unknown dtype */
  DET_ENONFINITE = 4,  /* an operand held Inf or NaN (device status) */
  DET_EHIP = 5,        /* the HIP runtime reported an error */
  DET_ERANGE = 6       /* a digit outside +-2^62 (device status) */
} det_status;

typedef enum { DET_F32 = 0, DET_BF16 = 1 } det_dtype;

/* Layout constants: 18, -298 and 2^19. */
int det_num_digits(void);
int det_lsb_exponent(void);
int64_t det_k_max(void);

/* Message for the calling thread's last failed call ("" if none). */
const char* det_last_error(void);

/*
 * det_gemm -- y = x * w^T, exact, rounded once to fp32 ("Usage" and "Method").
 *   dt           DET_F32 or DET_BF16 (both operands)
 *   x            element (m, k) at x[m*x_sm + k*x_sk], m < M, k < K
 *   w            element (n, k) at w[n*w_sn + k*w_sk], n < N, k < K
 *   y            fp32 output, element (m, n) at y[m*y_sm + n*y_sn]; must not
 *                overlap x or w
 *   M, N, K      sizes; M, N, K >= 0 and K <= 2^19.  K = 0 writes +0.0.
 * Returns DET_OK, DET_EINVAL, DET_EKLIMIT, DET_EDTYPE or DET_EHIP.
 */
det_status det_gemm(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk,
                    const void* w, int64_t w_sn, int64_t w_sk,
                    int64_t M, int64_t N, int64_t K,
                    float* y, int64_t y_sm, int64_t y_sn, void* stream);

/*
 * det_gemm_partial -- the raw digit array of x * w^T ("Usage": the partial of
 * a K-slice; "Method": digits of the long accumulator).
 *   Operands as for det_gemm.  acc is int64 [M][N][18], contiguous, written in
 *   full (K = 0 writes zeros).  Partials of disjoint K-slices combine with
 *   det_combine into exactly the partial of their union.
 */
det_status det_gemm_partial(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk,
                            const void* w, int64_t w_sn, int64_t w_sk,
                            int64_t M, int64_t N, int64_t K,
                            int64_t* acc, void* stream);

/*
 * Workspace variants.  det_gemm_ws and det_gemm_partial_ws compute exactly
 * what det_gemm and det_gemm_partial compute (bit-identical results) but
 * use a caller-provided device workspace: w is decoded into it once
 * (significands and exponent words, rows padded), and x one K block at a
 * time, which saves the GEMM kernels the decode of every element in every
 * output tile; a K range longer than 2^15 is run in blocks of 2^15 whose
 * exact digits are carried from block to block (in `acc` for the partial, in
 * the workspace for det_gemm), which keeps each block's slice of w in the L2
 * caches.
 *   workspace        device memory, 16-byte aligned, at least
 *                    det_gemm_workspace_bytes(dt, partial, M, N, K) bytes;
 *                    owned by the caller, overwritten by the call, and in use
 *                    until the call's work on `stream` has finished
 *   workspace_bytes  its size in bytes
 * det_gemm_workspace_bytes returns the size needed (0 when M, N or K is 0):
 * (partial ? 6 : 8) * roundup(N, 64) * roundup(K, 16) for w, plus
 * 8 * roundup(M, 2) * roundup(min(K, 2^15), 16) for x, plus 144 * M * N for
 * det_gemm_ws (partial = 0) when K > 2^15; for det_gemm_ws also the room of
 * the matrix-core path: roundup(32 (M + N) + 160, 256) +
 * 7 * (roundup(M, 128) + roundup(N, 128)) * roundup(K, 128) + 1024 (M + N) +
 * 16 * min(2^22, 2 M N), plus 16 * M * N when K > 2^14.  det_gemm_ws
 * given only the accumulator path's size (the sum without that last term)
 * runs the accumulator path.
 * Errors as for det_gemm, plus DET_EINVAL for a null, misaligned or too small
 * workspace.
 */
int64_t det_gemm_workspace_bytes(det_dtype dt, int partial, int64_t M, int64_t N, int64_t K);

det_status det_gemm_ws(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk,
                       const void* w, int64_t w_sn, int64_t w_sk,
                       int64_t M, int64_t N, int64_t K,
                       float* y, int64_t y_sm, int64_t y_sn,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * The matrix-core path of det_gemm_ws.  det_gemm only promises the exact sum
 * rounded once ("Method"), so for operands whose rows each span few binades
 * the sum may be formed with int8 matrix products instead of the digit
 * accumulator: each row of x and of w is scaled by a power of two to
 * integers below 2^(8S-2) in magnitude (S = 2..7), which are cut into S
 * signed 8-bit digits; the S^2 digit GEMMs run on the MFMA units with int32
 * sums, are added exactly in 128-bit integers and rounded once.  In a row
 * of x or w whose nonzero elements span more than 8S - 3 binades ("listed"),
 * the elements below the row's window ("tails") are left out of the digit
 * GEMMs; the outputs of listed rows and columns keep their exact 128-bit
 * sums, to which the tails' products are added one by one before the one
 * rounding.  A row with more than 256 tails, or more listed outputs than
 * 2^22, is recomputed on the accumulator path instead.  The results are
 * bit-identical to the accumulator path's for every input.
 *
 * The choice between the paths, and of S, depends on the spans of the
 * operands, which only the device sees; it is made on the device (a plan in
 * the workspace that every later kernel of the call reads), so the host
 * never waits: the call enqueues the kernels of every path the plan may
 * pick, and those not picked exit at once (a gated launch of the
 * accumulator takes up to 32 tiles per workgroup, so skipping it costs a
 * small grid's dispatch).  The rows the accumulator recomputes are counted
 * on the device too.
 *
 * det_set_gemm_path sets, for the whole process, which path det_gemm_ws
 * takes:
 *   DET_PATH_AUTO         (default) the matrix-core path is considered for
 *                         M*N*K >= 2^27 when the workspace has its room: the
 *                         call measures the spans (one pass over x and w)
 *                         and the device picks S, or the accumulator path,
 *                         by estimated time
 *   DET_PATH_AUTO_HOST    the same choice made by the host: the call waits
 *                         for the stream to read the 96-byte span histogram
 *                         (polling an event, so the thread keeps a CPU core
 *                         busy) and enqueues only the path it picks; not for
 *                         graph capture
 *   DET_PATH_ACCUMULATOR  always the digit accumulator
 *   DET_PATH_SLICES       always the matrix-core path (a too small workspace
 *                         is DET_EINVAL); `slices` = 2..7 fixes S, 0 lets the
 *                         device pick it
 * `slices` must be 0 or 2..7 (else DET_EINVAL); it is ignored by the other
 * paths.  det_gemm (no workspace) and the partials always use the
 * accumulator.
 *
 * det_last_gemm_plan reports the calling thread's last det_gemm or
 * det_gemm_ws call: the path taken (DET_PATH_ACCUMULATOR or DET_PATH_SLICES),
 * S (0 for the accumulator) and how many rows of x and of w were listed.
 * When the device made the plan it waits for that call's plan to be copied
 * back (an event wait); a call made under graph capture, or whose plan could
 * not be read, reports DET_PATH_AUTO and -1.  Null pointers are skipped.
 */
typedef enum { DET_PATH_AUTO = 0, DET_PATH_ACCUMULATOR = 1, DET_PATH_SLICES = 2, DET_PATH_AUTO_HOST = 3 } det_path;

det_status det_set_gemm_path(det_path path, int slices);

/* det_get_gemm_path -- the current process-wide setting of det_set_gemm_path
 * (path and slices); null pointers are skipped. */
void det_get_gemm_path(det_path* path, int* slices);

void det_last_gemm_plan(int* path, int* slices, int64_t* fallback_rows, int64_t* fallback_cols);

det_status det_gemm_partial_ws(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk,
                               const void* w, int64_t w_sn, int64_t w_sk,
                               int64_t M, int64_t N, int64_t K, int64_t* acc,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * det_gemm_noalloc -- det_gemm for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, result and errors as det_gemm, bit for bit;
 * it runs the pre-decoded digit accumulator of det_gemm_ws with the workspace
 * in a static device array of det_gemm_noalloc_max_bytes() = 64 MiB that the
 * library holds on every GPU it runs on until the process ends.  It allocates
 * nothing (no hipMalloc, no allocating library call) and never waits for the
 * device: the work is stream-ordered and asynchronous.
 * Limit: 8 roundup(N, 64) roundup(K, 16) + 8 roundup(M, 2) roundup(min(K, 2^15),
 * 16) (+ 144 M N when K > 2^15) must not exceed 64 MiB (for example
 * M = N = K = 2048), else DET_EINVAL before anything is enqueued.
 * All calls on one GPU share its array: calls whose work overlaps in time on
 * one GPU (on different streams, or from different threads without ordering)
 * race and give wrong results; the caller orders them.  No part of the array
 * needs to start at zero.
 */
det_status det_gemm_noalloc(det_dtype dt, const void* x, int64_t x_sm, int64_t x_sk,
                            const void* w, int64_t w_sn, int64_t w_sk,
                            int64_t M, int64_t N, int64_t K,
                            float* y, int64_t y_sm, int64_t y_sn, void* stream);

size_t det_gemm_noalloc_max_bytes(void);

/*
 * det_set_kernel_events -- for callers that time the GEMM kernel itself (the
 * benchmark): the calling thread's later det_gemm, det_gemm_ws,
 * det_gemm_noalloc, det_gemm_partial and det_gemm_partial_ws calls record
 * `start` (a hipEvent_t) on their stream just before the first launch of the
 * kernel that forms the products (the digit accumulator, or on the
 * matrix-core path the int8 digit GEMMs), and `stop` just after its last
 * launch; with K > 2^15 the interval also holds the per-block x decodes
 * between launches.  When the device picks the path (DET_PATH_AUTO on a
 * product that may take the matrix cores, DET_PATH_SLICES with slices = 0)
 * the interval wraps the accumulator's launches if the plan may pick that
 * path, else every digit-GEMM launch, picked or not: to time one kernel, fix
 * the path (DET_PATH_ACCUMULATOR, or DET_PATH_SLICES with S).  Calls that
 * launch no such kernel (an empty M or N) record nothing.  The events stay owned by the caller; null for either
 * turns its recording off.
 */
void det_set_kernel_events(void* start, void* stop);

/*
 * det_combine -- digit-wise int64 sum of accumulator arrays ("Usage" and
 * "Method": the partials of disjoint K ranges add digit by digit).
 *   parts        HOST array of `nparts` >= 1 device pointers, each to
 *                n_outputs*18 int64 digits
 *   out          device pointer to n_outputs*18 int64.  `out` may be equal
 *                to one or more of the parts (the same pointer; at most 32
 *                of them); a part that overlaps `out` without being equal
 *                to it is rejected with DET_EINVAL.
 *   n_outputs    number of accumulators (>= 0)
 * Precondition: every digit of every part, and every digit of the result,
 * lies within +-2^62 (room for the carries of rounding); with more than 32
 * parts the parts are added in groups of 32 and each group's running result
 * is stored in `out`, so it must lie in that range too.  Partials of GEMMs
 * whose K values add up to at most 2^30 always satisfy it.  A digit outside
 * the range is noted in the device status (DET_ERANGE from
 * det_device_status); the digits written are then unspecified.
 */
det_status det_combine(const int64_t* const* parts, int nparts, int64_t* out,
                       int64_t n_outputs, void* stream);

/*
 * det_finalize -- round each accumulator once to fp32 ("Method": the exact sum
 * rounded once to fp32).
 *   acc          n_outputs*18 int64 digits (any raw digits within +-2^62)
 *   y            n_outputs fp32 results, contiguous
 * A digit outside +-2^62 is noted in the device status (DET_ERANGE from
 * det_device_status); that output's value is then unspecified.
 */
det_status det_finalize(const int64_t* acc, float* y, int64_t n_outputs, void* stream);

/*
 * det_dot_partial -- raw digits of one exact dot product, for reductions of a
 * whole tensor such as a loss ("Method": every product exact, the sum in the
 * digits of one accumulator; the page's accumulator applied to one output).
 *   a, b         device operands of n elements each (bit patterns of dtype
 *                dt), element i at a[i * inc_a] and b[i * inc_b]
 *   inc_a, inc_b element increments (>= 0; 0 repeats one element)
 *   n            element count (>= 0)
 *   acc          device pointer to 18 int64 digits (8-byte aligned)
 *   accumulate   0: acc = the digits of sum_i a_i b_i; 1: acc += them
 * The digits are the same raw digits det_gemm_partial writes for the 1 x 1
 * GEMM of a and b (for n <= 2^19), so det_combine and det_finalize apply.
 * The digits are added into acc with 64-bit integer atomics: acc is in use
 * until the call's work on `stream` has finished, and calls that add into one
 * acc on different streams must not overlap.  At most 2^30 products may be
 * added into one acc over all calls (a dot product adds n): then every digit
 * stays within +-2^62.  An Inf or NaN element is noted in the device
 * status (DET_ENONFINITE from det_device_status); acc is then unspecified.
 * Returns DET_OK, DET_EINVAL, DET_EKLIMIT (more than 2^30 products in one
 * call), DET_EDTYPE or DET_EHIP.
 */
det_status det_dot_partial(det_dtype dt, const void* a, int64_t inc_a, const void* b, int64_t inc_b,
                           int64_t n, int64_t* acc, int accumulate, void* stream);

/*
 * det_sqdiff_partial -- raw digits of sum_i (a_i - b_i)^2, exactly: the
 * differences are never rounded, the sum is formed from the exact products
 * a_i a_i + b_i b_i - 2 a_i b_i (3 products per element).  b == NULL gives
 * sum_i a_i^2 (1 product per element; inc_b is ignored).  Arguments, digits,
 * limits and errors as for det_dot_partial.
 */
det_status det_sqdiff_partial(det_dtype dt, const void* a, int64_t inc_a, const void* b, int64_t inc_b,
                              int64_t n, int64_t* acc, int accumulate, void* stream);

/*
 * det_mse_grad -- the gradient of the exact mean squared error (the loss of
 * det_sqdiff_partial divided by n) with respect to its operands, for the
 * training step of the "Usage" section.  Elementwise, with no reduction:
 *     d  = RNE32(y_i - t_i)            (d = y_i without a target)
 *     gy = RNE32(RNE32(d * c) * g)     c = RNE32(2 / n), g = *g
 *     dy_i = gy,  dt_i = -gy           rounded to dt (nearest-even for bf16)
 * each fp32 step one IEEE operation, so the bits are fixed by the inputs.
 *   dt           DET_F32 or DET_BF16: the element type of y, t, dy and dt_out
 *   y, t         device operands of n elements, contiguous; t may be NULL
 *   c            2/n rounded to fp32 (by the caller, one IEEE division)
 *   g            device pointer to one fp32 value (the incoming gradient)
 *   dy, dt_out   device outputs of n elements; either may be NULL (not written)
 * Returns DET_OK, DET_EINVAL, DET_EDTYPE or DET_EHIP.
 */
det_status det_mse_grad(det_dtype dt, const void* y, const void* t, int64_t n, float c, const float* g, void* dy,
                        void* dt_out, void* stream);

/*
 * det_round_f32_to_bf16 -- round fp32 values to bf16 (nearest, ties to even),
 * used by the DetLinear backward of the "Usage" section to hand dY to a bf16
 * exact GEMM.  in: n fp32, out: n bf16 bit patterns; contiguous.  NaN stays NaN.
 */
det_status det_round_f32_to_bf16(const float* in, uint16_t* out, int64_t n, void* stream);

/*
 * det_check_finite -- set *flag (a device int32) to 1 if any element of the
 * [rows][cols] operand at p[r*s_row + c*s_col] is Inf or NaN; leaves it
 * untouched otherwise.  The caller zeroes the flag first.
 */
det_status det_check_finite(det_dtype dt, const void* p, int64_t rows, int64_t cols,
                            int64_t s_row, int64_t s_col, int32_t* flag, void* stream);

/*
 * Device status -- conditions only the kernels can see, reported after the
 * fact because every call is asynchronous.  Each GPU the library runs on
 * keeps a status word of its own, set by any call on any stream of that GPU
 * and cleared only here, like the sticky exception flags of IEEE 754:
 *   DET_ENONFINITE  an operand of det_gemm, det_gemm_ws, det_gemm_noalloc,
 *                   det_gemm_partial, det_gemm_partial_ws, det_dot_partial or
 *                   det_sqdiff_partial held an Inf or a NaN
 *   DET_ERANGE      a digit read by det_combine or det_finalize, or a digit
 *                   det_combine computed, lay outside +-2^62
 * The results of the call that set a condition are unspecified.
 *
 * det_device_status -- waits for `stream` (it blocks the calling thread),
 * reads the current device's word and, if `clear` is nonzero, clears it in
 * stream order after the read.  Returns DET_ENONFINITE if that condition is
 * set, else DET_ERANGE if that one is, else DET_OK (or DET_EHIP).  *flags,
 * unless null, gets 1 for non-finite plus 2 for range.  Work enqueued on
 * other streams and not ordered before the read may set the word after it,
 * and with `clear` a condition such work sets between the read and the
 * clear is lost: callers that use several streams order them first.
 *
 * det_device_status_word -- the current device's status word, for callers
 * that read it stream-ordered without waiting (a device copy, a kernel of
 * their own): four int32, [0] nonzero after a non-finite operand, [1] nonzero
 * after a digit out of range, [2] and [3] zero.  Null (see det_last_error) if
 * the device cannot be queried.  The caller may read it; only
 * det_device_status writes zeros to it.
 */
det_status det_device_status(void* stream, int clear, int* flags);

int32_t* det_device_status_word(void);

#ifdef __cplusplus
}
#endif

#endif /* DETGEMM_H */
