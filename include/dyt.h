/*
 * dyt.h - C ABI of the fused Dynamic Tanh (DyT) layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer, over an M x N row-major activation x with a scalar alpha and
 * per-column gamma and beta:
 *
 *   forward   y[i,j]   = gamma[j] * tanh(alpha * x[i,j]) + beta[j]
 *   backward  dx[i,j]  = dy[i,j] * gamma[j] * alpha * sech^2(alpha * x[i,j])
 *             dgamma[j] = sum_i dy[i,j] * tanh(alpha * x[i,j])
 *             dbeta[j]  = sum_i dy[i,j]
 *             dalpha    = sum_{i,j} dy[i,j] * gamma[j] * x[i,j] * sech^2(alpha x[i,j])
 *
 * with sech^2 = 1 - tanh^2. Source: the Liger-Kernel pull request "fix(dyt):
 * use a 1D grid and tile small-width rows" (#1616). Its Summary fixes the
 * behaviour this ABI keeps:
 *   - "Launch limit": any number of rows is accepted (a flat 1D grid; no
 *     65,535-block limit on rows).
 *   - "Small widths": narrow rows are packed several to a workgroup tile
 *     (whenever two or more fit a 4096-element tile, so every width up to
 *     256 qualifies); wider rows are cut into row segments, one per tile.
 *     The forward walks contiguous rows as one run of 16-byte vectors
 *     instead where that measured faster than these tiles (dyt_plan.flat).
 *   - "Padding": lanes past the end of the data are removed from the
 *     reductions after the arithmetic, so alpha = +inf cannot inject
 *     tanh(inf * 0) = NaN into dgamma, dbeta or dalpha.
 *   - "Precision": dalpha, dgamma and dbeta are returned in the parameter
 *     dtype; y and dx keep the dtype of x.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (memory of the current HIP
 *     device). Layout is contiguous row-major; the row stride is N elements
 *     (the *_strided entry points take explicit row strides).
 *     alpha, dalpha point to one element; gamma, beta, dgamma, dbeta to N.
 *   - x, dy, y, dx have the x dtype; alpha, gamma, beta, dalpha, dgamma,
 *     dbeta have the parameter dtype. Supported dtypes: DYT_F32, DYT_BF16
 *     and DYT_F16 for both, in any combination.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is only enqueued; no call synchronises. Outputs are valid once
 *     the stream reaches that point; inputs must stay unchanged until then.
 *   - Ownership: the caller owns every buffer; the library allocates no
 *     memory and keeps no state beyond immutable tables.
 *   - Outputs overwrite their buffers (they are not accumulated into) and
 *     must not overlap any input.
 *   - Alignment: every pointer must be aligned to its element size; the
 *     workspace must be 16-byte aligned. Activations at any element-aligned
 *     address, and rows of any length, use 16-byte vector memory access
 *     (gfx9 and later GPUs run global memory instructions in unaligned mode
 *     under ROCm), so alignment never changes the results.
 *   - Errors: every call returns DYT_OK (0) or a positive dyt_status.
 *     Arguments are validated before anything is enqueued, so on error no
 *     output is written. The library never prints and never throws.
 *     Faults during kernel execution surface at stream synchronisation.
 *   - Determinism: results are bitwise reproducible run to run. The
 *     parameter-gradient sums use a fixed summation order that depends only
 *     on (M, N, x dtype) (and, for the row-strided entry points, on whether
 *     they take the element-wise variant); no floating-point atomics.
 *   - Arithmetic is float32 throughout (accumulation included); bfloat16
 *     and float16 results are rounded to nearest even (values beyond the
 *     float16 range become +-inf). float32 subnormals are kept.
 */
#ifndef DYT_H_
#define DYT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DYT_ABI_VERSION 7

typedef enum dyt_dtype {
    DYT_F32 = 0,  /* IEEE binary32 */
    DYT_BF16 = 1, /* bfloat16: 8 exponent bits, 7 fraction bits */
    DYT_F16 = 2   /* IEEE binary16: 5 exponent bits, 10 fraction bits */
} dyt_dtype;

typedef enum dyt_status {
    DYT_OK = 0,
    DYT_ERR_INVALID_ARG = 1,         /* null pointer with a non-empty extent, M < 0, N < 0,
                                        size overflow, or an output overlapping an input */
    DYT_ERR_UNSUPPORTED_DTYPE = 2,   /* dtype code outside dyt_dtype */
    DYT_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < dyt_backward_workspace_size(...) */
    DYT_ERR_MISALIGNED = 4,          /* pointer not aligned to its element size, or
                                        workspace not 16-byte aligned */
    DYT_ERR_HIP = 5                  /* a HIP runtime call or kernel launch failed */
} dyt_status;

/*
 * Forward: y = gamma * tanh(alpha * x) + beta.
 *   x      [M, N] x_dtype, read
 *   alpha  [1]    param_dtype, read
 *   gamma  [N]    param_dtype, read
 *   beta   [N]    param_dtype, read
 *   y      [M, N] x_dtype, written
 * M == 0 or N == 0: nothing is enqueued and DYT_OK is returned (pointers may
 * then be NULL).
 * Launches that weight their workgroups by XCD (see dyt_xcd_hint) record the
 * XCD their first workgroup ran on in pinned host memory that the library
 * allocates once per device (256 bytes, on the first such launch outside
 * stream capture, kept until the process ends).
 */
int dyt_forward(const void* x, const void* alpha, const void* gamma, const void* beta,
                void* y, int64_t M, int64_t N, int x_dtype, int param_dtype,
                void* stream);

/*
 * Bytes of device workspace dyt_backward needs for this problem (a multiple
 * of 16; 0 when M == 0 or N == 0). Returns 0 as well for invalid arguments,
 * which dyt_backward then reports. Pure host function.
 */
size_t dyt_backward_workspace_size(int64_t M, int64_t N, int x_dtype, int param_dtype);

/*
 * Backward of the forward above, recomputing tanh(alpha * x) from x.
 *   x          [M, N] x_dtype, read
 *   dy         [M, N] x_dtype, read (upstream gradient of y)
 *   alpha      [1]    param_dtype, read
 *   gamma      [N]    param_dtype, read
 *   dx         [M, N] x_dtype, written
 *   dalpha     [1]    param_dtype, written (always, also when M*N == 0: 0)
 *   dgamma     [N]    param_dtype, written (zeros when M == 0)
 *   dbeta      [N]    param_dtype, written (zeros when M == 0)
 *   workspace  device scratch of workspace_bytes bytes, 16-byte aligned, no
 *              initial contents required; may be NULL when the required
 *              size is 0. Contents are undefined afterwards.
 * Equivalent to dyt_backward_partials followed by dyt_backward_finish on
 * the same stream (two kernels).
 */
int dyt_backward(const void* x, const void* dy, const void* alpha, const void* gamma,
                 void* dx, void* dalpha, void* dgamma, void* dbeta,
                 void* workspace, size_t workspace_bytes,
                 int64_t M, int64_t N, int x_dtype, int param_dtype,
                 void* stream);

/*
 * First backward pass alone: writes dx and, into the workspace, one float32
 * partial row [dgamma partials | dbeta partials | dalpha partial] per
 * workgroup (float32 accumulation; lanes past the end of the data are
 * removed after the arithmetic, so alpha = +inf cannot put
 * tanh(inf * 0) = NaN into the partials). The row layout depends only on
 * (M, N, x_dtype), never on pointer alignment. Arguments as dyt_backward.
 */
int dyt_backward_partials(const void* x, const void* dy, const void* alpha, const void* gamma,
                          void* dx, void* workspace, size_t workspace_bytes,
                          int64_t M, int64_t N, int x_dtype, int param_dtype, void* stream);

/*
 * Second backward pass alone: sums the partial rows that
 * dyt_backward_partials(M, N, x_dtype, ...) left in the workspace, column by
 * column in a fixed order, rounds to param_dtype and writes dgamma, dbeta
 * and dalpha. Arguments as dyt_backward; the workspace is only read.
 */
int dyt_backward_finish(const void* workspace, size_t workspace_bytes,
                        void* dalpha, void* dgamma, void* dbeta,
                        int64_t M, int64_t N, int x_dtype, int param_dtype, void* stream);

/*
 * Row-strided activations: the same forward and backward over tensors whose
 * rows are `ld` elements apart (ld >= N), e.g. an M x N block of a wider
 * buffer, so no copy is needed. Element (i, j) of x lives at x[i * ldx + j]
 * (likewise y with ldy, dy with lddy, dx with lddx). Any pitch takes the
 * 16-byte vector kernels, except rows short enough to be packed several to
 * a tile (N <= 2048) whose length N is not a multiple of 16 / sizeof(x):
 * those run the element-wise variant. The tiling is that of the contiguous
 * call, so with the vector kernels every partial row and the gradients'
 * summation order are too: the results equal those of dyt_forward /
 * dyt_backward on contiguous copies bit for bit. With the element-wise
 * variant y and dx still do; the gradients' rounding can differ, within the
 * stated tolerance. ld = N is the contiguous case.
 * Outputs must not overlap inputs anywhere between their first and last
 * element. Other arguments and conventions as dyt_forward / dyt_backward
 * (workspace size from dyt_backward_workspace_size(M, N, ...)); ld <= 0 or
 * ld < N is DYT_ERR_INVALID_ARG.
 */
int dyt_forward_strided(const void* x, int64_t ldx, const void* alpha, const void* gamma,
                        const void* beta, void* y, int64_t ldy, int64_t M, int64_t N,
                        int x_dtype, int param_dtype, void* stream);

int dyt_backward_strided(const void* x, int64_t ldx, const void* dy, int64_t lddy,
                         const void* alpha, const void* gamma, void* dx, int64_t lddx,
                         void* dalpha, void* dgamma, void* dbeta,
                         void* workspace, size_t workspace_bytes,
                         int64_t M, int64_t N, int x_dtype, int param_dtype, void* stream);

/*
 * Residual add fused with the layer (forward): the pre-norm block pattern
 * h = x + r ("x" the residual stream, "r" the branch output added to it)
 * followed by DyT of h, in one pass over memory:
 *
 *   h[i,j] = x[i,j] + r[i,j]            (rounded once to x_dtype)
 *   y[i,j] = gamma[j] * tanh(alpha * h[i,j]) + beta[j]
 *
 * y is computed from h as stored (rounded), so the pair (h, y) equals an
 * add followed by dyt_forward(h) bit for bit. It moves 4 M x N tensors
 * instead of the 5 of the two separate steps; the deepmd-kit pull request
 * "perf(pt): fuse the mixing-stack per-layer backward chain" (Motivation)
 * describes the HBM round trip of an intermediate that such fusion removes.
 *   x, r   [M, N] x_dtype, read
 *   alpha, gamma, beta as dyt_forward
 *   h      [M, N] x_dtype, written
 *   y      [M, N] x_dtype, written
 * h and y must not overlap each other or any input (no in-place h = x).
 * Other conventions, and M == 0 or N == 0, as dyt_forward.
 */
int dyt_forward_residual(const void* x, const void* r, const void* alpha, const void* gamma,
                         const void* beta, void* h, void* y, int64_t M, int64_t N,
                         int x_dtype, int param_dtype, void* stream);

/*
 * Backward of dyt_forward_residual: with dy the gradient of y and dres the
 * gradient reaching h through the residual stream,
 *
 *   dh[i,j] = dres[i,j] + dy[i,j] * gamma[j] * alpha * sech^2(alpha * h[i,j])
 *
 * (added in float32, rounded once to x_dtype) is the gradient of both x and
 * r; dgamma, dbeta and dalpha are those of dyt_backward(h, dy) - bit for bit
 * the same values, from the same partial rows. 4 M x N tensors move instead
 * of the 6 of dyt_backward followed by a separate add.
 *   h      [M, N] x_dtype, read (the h written by the forward)
 *   dy     [M, N] x_dtype, read
 *   dres   [M, N] x_dtype, read
 *   dh     [M, N] x_dtype, written
 * Other arguments, workspace (same size as dyt_backward's) and conventions
 * as dyt_backward; dh must not overlap any input.
 */
int dyt_backward_residual(const void* h, const void* dy, const void* dres, const void* alpha,
                          const void* gamma, void* dh, void* dalpha, void* dgamma, void* dbeta,
                          void* workspace, size_t workspace_bytes,
                          int64_t M, int64_t N, int x_dtype, int param_dtype, void* stream);

/*
 * First pass of dyt_backward_residual alone: writes dh and the partial rows
 * (identical to those of dyt_backward_partials(h, dy, ...)); finish with
 * dyt_backward_finish. Arguments as dyt_backward_residual.
 */
int dyt_backward_residual_partials(const void* h, const void* dy, const void* dres,
                                   const void* alpha, const void* gamma, void* dh,
                                   void* workspace, size_t workspace_bytes,
                                   int64_t M, int64_t N, int x_dtype, int param_dtype,
                                   void* stream);

/*
 * dyt_backward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The entry point allocates
 * nothing; the partial rows live in a static device array of
 * DYT_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on every GPU it
 * runs on until the process ends (its address is looked up once per device,
 * on the first call with that device current). Arguments, results, dtypes,
 * layout and the fixed summation order are those of dyt_backward (the same
 * kernels run, so the results equal dyt_backward's bit for bit).
 * Returns DYT_ERR_WORKSPACE_TOO_SMALL, before any HIP call, when
 * dyt_backward_workspace_size(M, N, ...) exceeds DYT_NOALLOC_SCRATCH_BYTES
 * (rows of up to 20,480 columns stay below 13 MiB; a single row of 2^22
 * float32 columns needs 32 MiB), and DYT_ERR_HIP if the array cannot be
 * located on the current device. Calls that overlap on one GPU (other
 * streams or host threads) share the array and race: serialise them.
 */
#define DYT_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int dyt_backward_noalloc(const void* x, const void* dy, const void* alpha, const void* gamma,
                         void* dx, void* dalpha, void* dgamma, void* dbeta,
                         int64_t M, int64_t N, int x_dtype, int param_dtype, void* stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* dyt_status_string(int status);

/* DYT_ABI_VERSION of the loaded library. */
int dyt_abi_version(void);

/*
 * Build id of the loaded library: 16 hex digits identifying the sources and
 * compiler flags it was built from (static storage; never NULL). The Python
 * binding refuses a library whose id differs from that of the sources next
 * to it.
 */
const char* dyt_build_id(void);

/*
 * XCD parity hint of the forward (performance only; results never depend on
 * it). The hardware places workgroup w of a launch on XCD (w + k) mod 8, k
 * fixed per hardware queue, and on MI355X the forward's workgroups on odd
 * XCDs stream more slowly, so the forward gives the larger share of its
 * tiles to the workgroups it expects on even XCDs. It learns k's parity
 * from the XCD its previous launch on the same stream started on.
 * dyt_xcd_hint returns that recorded XCD (0-7) for `stream` on the current
 * device, or -1 if none is recorded yet. dyt_set_xcd_flip_override forces
 * the parity for every later forward launch in the process (0 or 1; -1
 * returns to the recorded hint) and returns DYT_OK, or
 * DYT_ERR_INVALID_ARG for other values; it exists so that tests can run
 * both deals on any GPU.
 */
int dyt_xcd_hint(void* stream);
int dyt_set_xcd_flip_override(int flip);

/*
 * Launch geometry the library would use (for tests and reports; pure host
 * function, no HIP calls). dyt_get_plan describes the backward (pass 1 tiles,
 * grid and workspace layout; fwd_grid is the forward's grid), which depends
 * only on (M, N, x_dtype). Both directions take their tile size and grid
 * from a static table measured offline per (x dtype, row-length range), so
 * every plan is a pure function of the shape. vector_access selects which
 * kernel variant is described (non-zero: 16-byte vector access, which every
 * launch uses except the row-strided packed case named at
 * dyt_forward_strided; zero: that element-wise variant, vec = 1, same tiles
 * and workspace). Returns DYT_OK or the status the compute calls would
 * return for these sizes and dtypes.
 */
typedef struct dyt_plan {
    int32_t packed;        /* 1: tiles of >= 2 whole rows (N <= 2048); 0: row segments */
    int32_t vec;           /* elements per vector memory access (16 bytes, or 1) */
    int32_t slots;         /* vector slots per thread per tile */
    int32_t block;         /* threads per workgroup */
    int64_t rows_per_tile; /* packed: rows per tile; wide: 1 */
    int64_t tile_elems;    /* packed: rows_per_tile * N; wide: columns per row segment */
    int64_t col_blocks;    /* wide: row segments per row; packed: 1 */
    int64_t tiles;         /* number of tiles */
    int64_t fwd_grid;      /* forward workgroups */
    int64_t bwd_grid;      /* backward pass-1 workgroups = partial rows */
    int64_t ws_row;        /* floats between partial rows (a multiple of 32: 128-byte lines) */
    int64_t fin_grid;      /* backward pass-2 workgroups */
    int64_t ws_bytes;      /* workspace bytes this plan uses */
    int64_t flat;          /* forward: 1 if a contiguous launch walks the problem as one
                              run of 16-byte vectors instead of the tiles above (rows whose
                              length is a multiple of vec, at most 20480, that the tiles
                              fit poorly, and 2-byte x in packed tiles; rows that are
                              not: 2-byte x up to N + vec <= 3584,
                              float32 x up to N + vec <= 5120 when the tiles fit poorly);
                              row-strided launches use the tiles. 0 for the
                              element-wise variant (vector_access = 0). dyt_get_plan
                              reports the forward's value; the backward always tiles */
    int64_t flat_grid;     /* workgroups of that flat forward, 0 if flat = 0 */
    int64_t flat_aligned_only; /* 1 if that flat walk is taken only when x and y start
                              16-byte aligned or off that grid by the same amount (the
                              walk then starts at their first aligned element); 2-byte x
                              in packed tiles of one full slot, which the tiles serve
                              faster than an unaligned walk; 0 otherwise */
} dyt_plan;

int dyt_get_plan(int64_t M, int64_t N, int x_dtype, int param_dtype, int vector_access,
                 dyt_plan* out);

/*
 * The forward's geometry: the forward (plain and residual) tiles the problem
 * independently of the backward (it has no workspace), from its own row of
 * the tile table. Same struct; fwd_grid is the forward's grid and the
 * backward-only fields (bwd_grid, ws_row, fin_grid, ws_bytes) are 0.
 */
int dyt_get_forward_plan(int64_t M, int64_t N, int x_dtype, int param_dtype,
                         int vector_access, dyt_plan* out);

/*
 * The residual-fused forward's geometry (dyt_forward_residual), which has a
 * row of its own in the tile table and its own flat-walk rule (flat
 * whenever the tiles leave a slot empty). Same struct and conventions as
 * dyt_get_forward_plan, for the contiguous layout that entry point takes.
 */
int dyt_get_forward_residual_plan(int64_t M, int64_t N, int x_dtype, int param_dtype,
                                  dyt_plan* out);

#ifdef __cplusplus
}
#endif

#endif /* DYT_H_ */
