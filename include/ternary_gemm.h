/*
 * ternary_gemm.h -- C ABI of the MI355X (gfx950) ternary x int8 GEMM library
 * (libternary_gemm.so).
 *
 * Sources (cited by page title and section):
 *   [P10425] t27 pull request #10425, "t27c PTX backend: ternary x int8 GEMM
 *            kernel emitted by a .t27 spec (int8 mma.sync), ptx-run glue".
 *   [P10855] t27 pull request #10855, "spec(igla): hslm_bwd_ptx -- HSLM
 *            backward dX and dW as int8 tensor-core PTX written by t27".
 *
 * Stored ternary weights ("Wpacked").  W is a K x N matrix of weights in
 * {-1, 0, +1} kept as 2-bit codes, four per byte, one row of K/4 bytes per
 * output column n (N-major, the code index of (k, n) being n*K + k) [P10425
 * "What this adds"; P10855 PR body].  The code of (k, n) sits in byte
 * n*(K/4) + k/4 at bits 2*(k%4) and 2*(k%4)+1, the first code of a byte in the
 * least significant bits (the pages do not state the order inside a byte;
 * this is the reading taken).  A code c stands for the weight
 * (c & 1) - ((c >> 1) & 1): codes 0, 1, 2, 3 are 0, +1, -1, 0 [P10425 "What
 * this adds"; the same table appears as the byte-permute word 0x00FF0100 in
 * P10855 PR body].
 *
 * Conventions shared by every call:
 *   - All matrix arguments are DEVICE pointers to dense row-major storage with
 *     no padding between rows; the caller owns them.  The library allocates,
 *     frees, copies and retains nothing (the dX calls that take a workspace
 *     borrow the caller's device memory for the duration of the call).
 *   - No alignment beyond the element size is required; aligned bases and
 *     row lengths that are multiples of 16 take the fast load path.
 *   - Each call validates its arguments on the host first.  On any error it
 *     returns a negative status, launches nothing and leaves every output
 *     untouched.
 *   - On success the work is enqueued on `stream` (NULL: the default stream)
 *     and the call returns without waiting.  Faults that only show while the
 *     kernel runs surface at the caller's next synchronisation.
 *   - Results are exact: integer sums in int32, each output reduced over the
 *     whole contraction in a fixed order with no atomics: inside one
 *     workgroup, or, on the workspace path of dX, as per-workgroup partial
 *     sums added in split order by a second kernel.  Integer addition is
 *     exact, so every path and every repeated call gives identical bits.
 *   - Calls are thread-safe; concurrent calls on different streams may run at
 *     the same time as long as their outputs do not overlap.
 */
#ifndef TERNARY_GEMM_H
#define TERNARY_GEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum tgemm_status {
    TGEMM_OK = 0,
    TGEMM_ERR_NULL = -1,   /* a required pointer is NULL                        */
    TGEMM_ERR_DIM = -2,    /* a dimension is < 1, or a size does not fit        */
    TGEMM_ERR_PACK = -3,   /* the packed dimension K is not a multiple of 4     */
    TGEMM_ERR_BOUND = -4,  /* the contraction is longer than the exact-int32 bound */
    TGEMM_ERR_ALIAS = -5,  /* the output overlaps an input                       */
    TGEMM_ERR_HIP = -6,    /* the HIP runtime reported an error at launch        */
    TGEMM_ERR_KIND = -7,   /* the output kind of a scaled call is not one of
                              TGEMM_OUT_F32, TGEMM_OUT_BF16, or the input kind
                              of a quantizer call not TGEMM_IN_F32,
                              TGEMM_IN_BF16                                   */
    TGEMM_ERR_SCRATCH = -8 /* ternary_gemm_s8_dx_noalloc: the split needs more
                              than TGEMM_STATIC_SCRATCH_BYTES of scratch      */
} tgemm_status;

/* Longest contraction for which every int32 result is exact whatever the
 * inputs.  Ternary x int8 (forward, dX): |sum| <= 128 * L must fit int32,
 * L <= floor((2^31 - 1) / 128) [P10425 "What this adds", invariant "i32
 * overflow bound"].  int8 x int8 (dW): L <= floor((2^31 - 1) / 128^2) = 131071
 * [P10855 PR body, kernel 2, "k <= 131071"]. */
#define TGEMM_TERNARY_MAX_CONTRACTION 16777215LL
#define TGEMM_INT8_MAX_CONTRACTION 131071LL

/*
 * Forward product [P10425 "What this adds"]:
 *     C[m][n] = sum_{k<K} A[m][k] * w(k, n)
 *   A        int8    [M][K]
 *   Wpacked  uint8   [N][K/4]   (stored ternary weights, layout above)
 *   C        int32   [M][N]     (written, never read)
 * Requires M, N, K >= 1, K % 4 == 0 (TGEMM_ERR_PACK otherwise) and
 * K <= TGEMM_TERNARY_MAX_CONTRACTION (TGEMM_ERR_BOUND).
 */
int ternary_gemm_s8(const int8_t *A, const uint8_t *Wpacked, int32_t *C,
                    int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * dX = dC x W^T with the same stored ternary W as the forward product
 * [P10855 PR body, kernel 1 "hslm_dx_s8"]:
 *     dX[m][k] = sum_{n<N} dC[m][n] * w(k, n)
 *   dC       int8    [M][N]
 *   Wpacked  uint8   [N][K/4]   (the forward call's buffer, unchanged)
 *   dX       int32   [M][K]     (written, never read)
 * Requires M, N, K >= 1, K % 4 == 0 (TGEMM_ERR_PACK) and
 * N <= TGEMM_TERNARY_MAX_CONTRACTION (TGEMM_ERR_BOUND).
 */
int ternary_gemm_s8_dx(const int8_t *dC, const uint8_t *Wpacked, int32_t *dX,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * dW = A^T x dC, int8 x int8 -> int32, summed over the M rows
 * [P10855 PR body, kernel 2 "hslm_dw_s8"]:
 *     dW[k][n] = sum_{m<M} A[m][k] * dC[m][n]
 *   A        int8    [M][K]
 *   dC       int8    [M][N]
 *   dW       int32   [K][N]     (written, never read)
 * Requires M, N, K >= 1 and M <= TGEMM_INT8_MAX_CONTRACTION (TGEMM_ERR_BOUND).
 * K need not be a multiple of 4 (no packed operand).
 */
int ternary_gemm_s8_dw(const int8_t *A, const int8_t *dC, int32_t *dW,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * Scaled outputs: the integer product followed by its dequantization, fused
 * into the kernels' stores.  The pages leave the scales to the host: the
 * activations are quantized per row for dX and X and dY per column for dW
 * [P10855 PR body]; the forward takes the same per-row activation scale, and
 * the ternary weights one scale for the whole matrix (the reading taken).
 * Each output element is
 *     y = (float(acc) * row_scale[row]) * col_scale
 * where acc is the exact int32 result of the plain call, the int32 -> float
 * conversion and each product are IEEE single precision rounded to nearest
 * even, in that order, and col_scale is the weight scale (forward, dX) or
 * dc_col_scale[n] (dW).  TGEMM_OUT_F32 stores y as float; TGEMM_OUT_BF16
 * stores y rounded to the nearest bfloat16, ties to even (a NaN stays a
 * quiet NaN), as uint16 bit patterns, which halves the bytes written.
 * Scale vectors are DEVICE float arrays; output element counts and layouts
 * are those of the plain calls.  Besides the plain calls' checks, a NULL
 * scale vector returns TGEMM_ERR_NULL, an output kind other than the two
 * below TGEMM_ERR_KIND, and an output overlapping a scale vector
 * TGEMM_ERR_ALIAS.
 */
#define TGEMM_OUT_F32 1
#define TGEMM_OUT_BF16 2

/* forward: Y[m][n] = (float(C[m][n]) * a_row_scale[m]) * w_scale;
 * a_row_scale float [M]. */
int ternary_gemm_s8_scaled(const int8_t *A, const uint8_t *Wpacked, const float *a_row_scale,
                           float w_scale, void *Y, int out_kind,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* dX: Y[m][k] = (float(dX[m][k]) * dc_row_scale[m]) * w_scale;
 * dc_row_scale float [M]. */
int ternary_gemm_s8_dx_scaled(const int8_t *dC, const uint8_t *Wpacked, const float *dc_row_scale,
                              float w_scale, void *dX, int out_kind,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * dX with a workspace, for few rows and long rows of Wpacked (the backward
 * of a decode-sized batch, [P10855 "Measured"]: 27 rows).  Same products,
 * arguments, checks and results as ternary_gemm_s8_dx and
 * ternary_gemm_s8_dx_scaled; in addition the caller lends `workspace`, a
 * DEVICE buffer of `workspace_bytes` bytes.  When M <= 32, N % 64 == 0,
 * K % 256 == 0, dC and Wpacked are 16-byte aligned and K / 256 column
 * blocks are too few to fill the chip, the contraction is split across
 * workgroups: each writes its int32 partial sums to the workspace and a
 * second kernel adds them in split order, which is faster when each W row is
 * long (27 x 16384 x 16384: about 32 against 46 us).  The workspace must then hold
 * ternary_gemm_dx_workspace() bytes and be 16-byte aligned; a NULL, smaller
 * or unaligned workspace runs the one-pass kernels instead, with the same
 * results.  The workspace's contents on entry do not matter and are garbage
 * afterwards; it is in use until the call completes on `stream`, so calls
 * that may overlap need workspaces of their own.  A workspace overlapping an
 * input, the output or the scale vector returns TGEMM_ERR_ALIAS, a negative
 * workspace_bytes TGEMM_ERR_DIM.
 */
int ternary_gemm_s8_dx_ws(const int8_t *dC, const uint8_t *Wpacked, int32_t *dX,
                          int64_t M, int64_t N, int64_t K, void *workspace,
                          int64_t workspace_bytes, hipStream_t stream);
int ternary_gemm_s8_dx_scaled_ws(const int8_t *dC, const uint8_t *Wpacked, const float *dc_row_scale,
                                 float w_scale, void *dX, int out_kind,
                                 int64_t M, int64_t N, int64_t K, void *workspace,
                                 int64_t workspace_bytes, hipStream_t stream);

/*
 * dX that allocates nothing, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same product, arguments, checks and results as
 * ternary_gemm_s8_dx_ws, with the workspace taken from a static device
 * buffer of TGEMM_STATIC_SCRATCH_BYTES that the library holds on each device
 * it runs on until the process ends (its address is looked up once per
 * device, on the device's first call).  When the contraction split applies
 * and needs more than that buffer (ternary_gemm_dx_workspace() bytes), the
 * call returns TGEMM_ERR_SCRATCH and launches nothing; without a split it
 * runs the one-pass kernels.  The call itself allocates nothing: no
 * hipMalloc, hipFree or allocating library routine.  Every call on a device
 * shares that device's buffer, whose contents on entry do not matter: calls
 * that may overlap on one device (two streams, two threads) race on it and
 * must be serialized by the caller.
 */
#define TGEMM_STATIC_SCRATCH_BYTES (8 << 20)
int ternary_gemm_s8_dx_noalloc(const int8_t *dC, const uint8_t *Wpacked, int32_t *dX,
                               int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Workspace bytes the dX calls above use for these dimensions when the
 * inputs' base alignment is `align` bytes (the smallest power-of-two
 * alignment of dC and Wpacked; <= 0 counts as 1): written to *bytes, 0 when
 * the one-pass kernels run anyway.  Returns TGEMM_OK, TGEMM_ERR_NULL for a
 * NULL `bytes`, or the status a dX call would return for the dimensions. */
int ternary_gemm_dx_workspace(int64_t M, int64_t N, int64_t K, int64_t align, int64_t *bytes);

/* dW: Y[k][n] = (float(dW[k][n]) * a_col_scale[k]) * dc_col_scale[n];
 * a_col_scale float [K], dc_col_scale float [N]. */
int ternary_gemm_s8_dw_scaled(const int8_t *A, const int8_t *dC, const float *a_col_scale,
                              const float *dc_col_scale, void *dW, int out_kind,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * The steps before the product (the pages give the stored format and where
 * the activation scales go; the rules below are the readings taken).
 *
 * Packing the trainer's ternary weights [P10425 "What this adds": code
 * table; P10855 PR body: wiring the trainer is left for later]:
 *     Wpacked[n][k/4] bits 2(k%4), 2(k%4)+1  <-  code of Wt[n][k]
 * with code 1 for w > 0, 2 for w < 0, 0 for w == 0 (so {-1, 0, +1} map to
 * their codes and code 3 is never written).
 *   Wt       int8   [N][K]     (row n: the weights of output column n, the
 *                               layout of a linear layer's weight; device)
 *   Wpacked  uint8  [N][K/4]   (written, never read; device)
 * Requires N, K >= 1 and K % 4 == 0 (TGEMM_ERR_PACK); an output overlapping
 * the input returns TGEMM_ERR_ALIAS.
 */
int ternary_pack_weights(const int8_t *Wt, uint8_t *Wpacked, int64_t N, int64_t K, hipStream_t stream);

/*
 * Symmetric int8 quantization of activations, with one scale per row
 * (ternary_quantize_rows: the forward's A and dX's dC) or per column
 * (ternary_quantize_cols: dW's A and dC) [P10855 PR body, the host's
 * scales: per row for dX, per column of X and dY for dW]:
 *     s = max |x| / 127                       over the row or column
 *     q = clamp(rint(x / s), -127, 127)       (q = 0 where s == 0)
 * each step in IEEE single precision rounded to nearest even (rint: ties to
 * even).  The scale is the one the scaled calls above take, so that
 * q * s approximates x to within half a step.
 *   X      [R][C] float32 (TGEMM_IN_F32) or bfloat16 bit patterns
 *          (TGEMM_IN_BF16), finite values (device)
 *   Q      int8  [R][C] (written; device)
 *   scale  float [R] (rows) or [C] (cols) (written; device; the column
 *          variant also uses it as its running maximum, so it must not be
 *          read by other work until the call completes)
 * A NULL pointer returns TGEMM_ERR_NULL, another input kind TGEMM_ERR_KIND,
 * R or C < 1 TGEMM_ERR_DIM, overlapping buffers TGEMM_ERR_ALIAS.
 */
#define TGEMM_IN_F32 1
#define TGEMM_IN_BF16 2
int ternary_quantize_rows(const void *X, int in_kind, int8_t *Q, float *scale, int64_t R, int64_t C,
                          hipStream_t stream);
int ternary_quantize_cols(const void *X, int in_kind, int8_t *Q, float *scale, int64_t R, int64_t C,
                          hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *ternary_gemm_status_str(int status);

/*
 * Launch plan the library would use for a call, computed on the host without
 * touching the device (for tests and tooling).  op: 0 forward, 1 dX, 2 dW.
 * Fills the output tile (rows x cols of the row-major output computed at a
 * time by one workgroup), the number of tiles, the number of workgroups
 * launched and the most tiles any one of them computes (1 for the one-tile
 * kernels; persistent kernels loop over several), the tile columns per band
 * of the one-tile kernels' workgroup -> tile order, whether the fast
 * (vector-load) path applies given the base alignments passed in `align`
 * (the smallest power-of-two alignment of the input pointers, in bytes),
 * which kernel runs (TGEMM_KERNEL_*), and that kernel's threads and LDS bytes
 * per workgroup.  The plan is that of the calls without a workspace.
 * Returns TGEMM_OK, or the status the real call would return for these
 * dimensions (pointer checks excepted).
 */
#define TGEMM_KERNEL_TILED 0   /* one 4-wave workgroup per output tile          */
#define TGEMM_KERNEL_SPLIT 2   /* dW, and dX with at most 256 tiles, on 128 x 144
                                  tiles: the tile's contraction split between
                                  two 4-wave halves of one workgroup          */
#define TGEMM_KERNEL_STREAM 3  /* forward (K % 64 == 0) and dX (N % 64 == 0,
                                  K % 16 == 0) on 16-byte aligned A or dC and
                                  4-byte aligned Wpacked, 32-bit offsets, at
                                  least 256 tiles of 512 x 144 (forward) or
                                  512 x 160 (dX): one persistent 8-wave
                                  workgroup per CU, operands loaded straight
                                  into LDS                                    */
#define TGEMM_KERNEL_SKINNY 4  /* forward with M <= 32, K % 64 == 0, 16-byte
                                  aligned A and Wpacked; dX with M <= 32,
                                  N % 64 == 0, K % 16 == 0, 16-byte aligned dC
                                  and Wpacked aligned for its row loads: one
                                  8-wave workgroup per 16, 32 or 64 output
                                  columns and all M rows, its waves splitting
                                  the contraction                             */

typedef struct tgemm_plan {
    int64_t out_rows, out_cols, contraction;
    int32_t tile_rows, tile_cols;
    int64_t tiles;
    int64_t workgroups;
    int64_t tiles_per_workgroup;
    int32_t band_cols;
    int32_t threads_per_workgroup;
    int32_t lds_bytes;
    int32_t fast_path;
    int32_t kernel;
    int32_t xcds;              /* XCDs of the machine planned for            */
} tgemm_plan;

int ternary_gemm_plan(int op, int64_t M, int64_t N, int64_t K, int64_t align,
                      tgemm_plan *plan);

/*
 * The same plan for a machine with `cus` compute units in `xcds` XCDs (cus a
 * multiple of xcds; TGEMM_ERR_DIM otherwise).  ternary_gemm_plan plans for
 * MI355X (256 CUs, 8 XCDs); the calls plan for the device they run on, whose
 * counts ternary_gemm_machine reports (it queries the current HIP device
 * once and keeps the answer; TGEMM_ERR_HIP if there is none).
 */
int ternary_gemm_plan_on(int op, int64_t M, int64_t N, int64_t K, int64_t align,
                         int32_t cus, int32_t xcds, tgemm_plan *plan);
int ternary_gemm_machine(int32_t *cus, int32_t *xcds);

/*
 * Output tile that workgroup `workgroup` computes in its iteration
 * `iteration` (0 .. tiles_per_workgroup - 1) under a plan: a host mirror of
 * the kernels' own workgroup -> tile order.  That order gives each of the
 * chip's eight L2 slices (XCDs; workgroup b runs on XCD b % 8) a contiguous
 * run of tiles, row by row (inside bands of band_cols tile columns for the
 * one-tile kernels), so tiles in flight together on one XCD share input rows
 * and columns in its L2.  Writes the tile's first output row and column.
 * Returns TGEMM_OK, or TGEMM_ERR_DIM if the workgroup is out of range or
 * computes no tile in that iteration.
 */
int ternary_gemm_tile_of(const tgemm_plan *plan, int64_t workgroup, int64_t iteration,
                         int64_t *row0, int64_t *col0);

#ifdef __cplusplus
}
#endif

#endif /* TERNARY_GEMM_H */
