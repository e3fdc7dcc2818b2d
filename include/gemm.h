/*
 * gemm.h -- C ABI of the MI355X (gfx950) dense half-precision GEMM library
 * (libdhpt_gemm.so).  Plain C types only; no allocation, no host
 * synchronisation, no state kept between calls.
 *
 * The operation (gemm_run) is the alpha = 1, beta = 0 case of
 * C <- alpha*A*B + beta*C in which the old C is never read, on row-major
 * A [M,K], B [K,N] and C [M,N] ("GEMM From Naive CUDA to Tensor Cores",
 * opening section; its section "Layout is part of the type" lists what the
 * contract must pin down: logical shapes, storage order, leading dimensions,
 * alignment and the input/accumulator/output types):
 *
 *     C[i*ldc + j] = sum_{k=0}^{K-1} A[i*lda + k] * B[k*ldb + j]
 *                    for 0 <= i < M, 0 <= j < N.
 *
 * The products of the half-precision inputs are accumulated in fp32 (the
 * FP16-in, FP32-accumulate contract the Ada tensor-core GEMM write-up states
 * at its start), then converted once to the output type (fp32 as is; fp16 and
 * bf16 by IEEE round-to-nearest-even).
 *
 * 8-bit float inputs (the GEMM_E4M3_* and GEMM_E5M2_* dtypes) extend the same
 * contract to the E4M3 and E5M2 formats of the OCP 8-bit floating point
 * specification (OFP8), the 8-bit float the Ada write-up's precision notes
 * leave as the next step: products accumulated in fp32, one rounding to the
 * output type.  Both B layouts are accepted.
 */
#ifndef DHPT_GEMM_H
#define DHPT_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input/output type pair.  A and B always share the input type. */
typedef enum {
    GEMM_F16_F32 = 0,   /* fp16 A, B -> fp32 C */
    GEMM_F16_F16 = 1,   /* fp16 A, B -> fp16 C */
    GEMM_BF16_F32 = 2,  /* bf16 A, B -> fp32 C */
    GEMM_BF16_BF16 = 3, /* bf16 A, B -> bf16 C */
    /* 8-bit float A, B (1-byte elements, OFP8 E4M3 / E5M2) */
    GEMM_E4M3_F32 = 4,  /* E4M3 A, B -> fp32 C */
    GEMM_E4M3_F16 = 5,  /* E4M3 A, B -> fp16 C */
    GEMM_E4M3_BF16 = 6, /* E4M3 A, B -> bf16 C */
    GEMM_E5M2_F32 = 7,  /* E5M2 A, B -> fp32 C */
    GEMM_E5M2_F16 = 8,  /* E5M2 A, B -> fp16 C */
    GEMM_E5M2_BF16 = 9  /* E5M2 A, B -> bf16 C */
} gemm_dtype_t;

/* Status codes.  Every error is returned before anything is enqueued. */
enum {
    GEMM_OK = 0,
    GEMM_ERR_DIM = -1,      /* M, N or K negative */
    GEMM_ERR_LD = -2,       /* lda < K, ldb < N or ldc < N (or a negative ld) */
    GEMM_ERR_NULL = -3,     /* C null with M*N > 0, or A/B null with M*N*K > 0 */
    GEMM_ERR_DTYPE = -4,    /* dtype not one of gemm_dtype_t */
    GEMM_ERR_ALIAS = -5,    /* C's byte range overlaps A's or B's */
    GEMM_ERR_RANGE = -6,    /* a dimension >= 2^31, a leading dimension > 2^40, an
                               operand spanning more than 2^47 elements, or more
                               than 2^31-1 output tiles */
    GEMM_ERR_LAUNCH = -7,   /* the HIP runtime rejected the kernel launch */
    GEMM_ERR_ALIGN = -8,    /* a pointer not aligned to its element size */
    GEMM_ERR_INSTANCE = -9, /* gemm_run_instance: unknown id, or the instance
                               cannot handle this shape/alignment */
    GEMM_ERR_LAYOUT = -10,  /* gemm_run_ex: b_layout not one of gemm_layout_t */
    GEMM_ERR_WORKSPACE = -11 /* gemm_run_ws: workspace null, smaller than
                                gemm_workspace_size() or not 256-byte aligned */
};

/* Storage order of B for gemm_run_ex (A and C are always row-major). */
typedef enum {
    GEMM_B_ROW_MAJOR = 0,   /* B(k,j) at B[k*ldb + j], ldb >= N (gemm_run's layout) */
    GEMM_B_COL_MAJOR = 1    /* B(k,j) at B[j*ldb + k], ldb >= K: B stored column-major,
                               i.e. its N x K transpose row-major -- the "TN" layout the
                               Ada tensor-core GEMM write-up builds on (its operand-
                               layout choice: A row-major, B column-major) */
} gemm_layout_t;

/*
 * gemm_run -- enqueue C = A.B on `stream`.
 *
 *   M, N, K    logical sizes (A is M x K, B is K x N, C is M x N).
 *   dtype      a gemm_dtype_t value.
 *   A, lda     device pointer to row-major A; element (i,k) at A[i*lda + k]
 *              (16-bit elements; 8-bit for the 8-bit dtypes), lda >= K.
 *   B, ldb     device pointer to row-major B; element (k,j) at B[k*ldb + j],
 *              ldb >= N.
 *   C, ldc     device pointer to row-major C; element (i,j) at C[i*ldc + j]
 *              (4-byte elements for fp32 output, 2-byte otherwise), ldc >= N.
 *   stream     a hipStream_t cast to void*; NULL means the null stream.
 *
 * Ownership: the caller allocates A, B and C on the current HIP device and
 * keeps them alive until the enqueued work completes.  The library allocates
 * nothing and reads A and B only.  It writes exactly the M x N elements of C;
 * the padding columns j >= N of each C row (and everything else) are never
 * touched, and the old contents of C are never read.
 *
 * Sizes: M == 0 or N == 0 is a successful no-op.  K == 0 writes zeros to the
 * M x N region (the product of an M x 0 and a 0 x N matrix).
 *
 * Alignment: only natural element alignment is required (2 bytes for 16-bit
 * A and B, none for 8-bit ones; 4 or 2 bytes for C).  Whole tiles (256x256,
 * 128x128 or 64x64, chosen by the number of tiles and K) with K a multiple of
 * 64 (128 for 8-bit inputs) run without edge code; other shapes with N a
 * multiple of 8 (16 for 8-bit inputs; any N with column-major B) run with
 * clamped edge loads and a zero-filled last k-slice; any other N runs on a
 * fully masked fallback, and so do leading dimensions so large that one
 * tile's rows of A (or of column-major B), or one 128-byte slice's rows of
 * row-major B, span 2 GiB or more (about 4.2 million 16-bit elements per row
 * at 256x256 tiles): the faster kernels address their copies as 31-bit
 * offsets from a per-tile base.
 *
 * Returns GEMM_OK once the kernel is enqueued (asynchronous: device faults
 * surface at the caller's next synchronisation), or a GEMM_ERR_* code.
 */
int gemm_run(int64_t M, int64_t N, int64_t K, int dtype,
             const void* A, int64_t lda, const void* B, int64_t ldb,
             void* C, int64_t ldc, void* stream);

/*
 * gemm_run_ex -- the general form with a fused epilogue, enqueued on `stream`:
 *
 *     C[i*ldc + j] <- act( alpha * sum_k A[i*lda + k] * B(k, j)
 *                          + beta * C[i*ldc + j] + bias[j] )
 *
 * for 0 <= i < M, 0 <= j < N: the general C <- alpha*A*B + beta*C that "GEMM
 * From Naive CUDA to Tensor Cores" opens with, plus the per-column bias and
 * ReLU that the Ada tensor-core GEMM write-up folds into the epilogue (its
 * remark on the fused bias + ReLU epilogue).  The dot product is accumulated in fp32;
 * the epilogue runs in fp32 on that accumulator (alpha * acc, then
 * + beta * C_old as a fused multiply-add, then + bias[j], then ReLU) and the
 * result is rounded once to the output type.
 *
 *   b_layout   a gemm_layout_t value: B(k, j) = B[k*ldb + j] (row-major,
 *              ldb >= N) or B[j*ldb + k] (column-major, ldb >= K).
 *   alpha      scale of the product.
 *   beta       scale of the old output.  With beta == 0 the old contents of
 *              C are never read (they may hold anything, NaN included);
 *              otherwise C is read in its output type before it is written.
 *   bias       device pointer to N fp32 values (4-byte aligned), or NULL for
 *              no bias.  Must not overlap C (GEMM_ERR_ALIAS).
 *   relu       nonzero: act(x) = max(x, 0) (a NaN stays NaN); zero: identity.
 *
 * Other arguments, ownership, sizes and errors as gemm_run, plus
 * GEMM_ERR_LAYOUT.  K == 0 gives C = act(beta*C + bias).  With b_layout
 * GEMM_B_ROW_MAJOR, alpha == 1, beta == 0, bias == NULL and relu == 0 the
 * call is gemm_run, bit for bit.
 */
int gemm_run_ex(int64_t M, int64_t N, int64_t K, int dtype, int b_layout,
                const void* A, int64_t lda, const void* B, int64_t ldb,
                void* C, int64_t ldc, float alpha, float beta,
                const float* bias, int relu, void* stream);

/*
 * gemm_workspace_size -- bytes of device workspace gemm_run_ws uses (a
 * constant of the library, 4096).
 *
 * gemm_run_ws -- gemm_run_ex with a caller-owned workspace, which lets the
 * library schedule the output tiles dynamically: with at least two 256x256
 * tiles per compute unit (16-bit inputs), it launches one workgroup per CU
 * and each takes tiles from shared counters until none is left, first from
 * the queue of the XCD it runs on (the tiles the one-workgroup-per-tile
 * launch deals to that XCD, in the same L2-friendly order), then from the
 * other XCDs' queues -- the persistent kernel of "The Asynchronous Kernel:
 * Tensor Cores & TMA", section "Keeping the line busy", which removes the
 * tail left by XCDs running at different clocks.  Other shapes run exactly
 * as gemm_run_ex would.  The result is bit for bit that of gemm_run_ex (the
 * same per-tile arithmetic; only the order in which tiles are visited
 * changes).
 *
 *   workspace        device pointer, 256-byte aligned, at least
 *                    gemm_workspace_size() bytes, on the current device.  It
 *                    must hold zeros before its first use (e.g. hipMemset
 *                    once after allocation); every call leaves it zeroed when
 *                    its kernel has finished.  The caller owns it.  Calls
 *                    that may run at the same time (different streams, or a
 *                    graph replayed concurrently) must use different
 *                    workspaces; calls ordered on one stream may share one.
 *                    It must not overlap A, B, C or the bias (GEMM_ERR_ALIAS).
 *   workspace_bytes  its size in bytes.
 *
 * Other arguments, ownership and status codes as gemm_run_ex, plus
 * GEMM_ERR_WORKSPACE.  No allocation, no host synchronisation; the first call
 * on a device queries that device's compute-unit count (kept for later
 * calls).
 */
int64_t gemm_workspace_size(void);

int gemm_run_ws(int64_t M, int64_t N, int64_t K, int dtype, int b_layout,
                const void* A, int64_t lda, const void* B, int64_t ldb,
                void* C, int64_t ldc, float alpha, float beta,
                const float* bias, int relu, void* workspace,
                int64_t workspace_bytes, void* stream);

/*
 * gemm_run_noalloc -- gemm_run_ws for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, bit for bit, with the persistent
 * kernels' scheduler words kept in a 4 KiB array of the library's own device
 * memory instead of a caller's workspace.  It calls no hipMalloc, hipFree or
 * other allocating routine.
 *
 * Limit and sharing: the array (4096 bytes, the most the scheduler uses; a
 * call needing more would be refused with GEMM_ERR_WORKSPACE) exists once
 * per device, for the life of the process, and every call on that device
 * uses it.  Calls that overlap in time on one device (different streams,
 * concurrent graph replays) race on it and must not be issued; calls ordered
 * on one stream are safe.  When the persistent kernel is selected, a small
 * kernel first clears the array on `stream`.  The first call on a device
 * looks the array's device address up (hipGetSymbolAddress) and keeps it:
 * make that first call outside any stream capture; later calls can be
 * captured into a HIP graph and replayed.
 *
 * Arguments, ownership and status codes as gemm_run_ex; GEMM_ERR_LAUNCH also
 * when the array's device address cannot be obtained.
 */
int gemm_run_noalloc(int64_t M, int64_t N, int64_t K, int dtype, int b_layout,
                     const void* A, int64_t lda, const void* B, int64_t ldb,
                     void* C, int64_t ldc, float alpha, float beta,
                     const float* bias, int relu, void* stream);

/*
 * gemm_splitk_workspace_size -- bytes of workspace gemm_run_splitk needs for
 * an M x N x K problem cut into `splits` pieces of K: one fp32 256 x 256
 * partial tile per output tile of 256 x 256 and per piece,
 * ceil(M/256) * ceil(N/256) * pieces * 262144 bytes, where pieces =
 * ceil(K / Kc) with Kc = ceil(K / splits) rounded up to a multiple of 64
 * (so pieces <= splits; 8-bit inputs cut pieces of a multiple of 128, never
 * more of them, so the same size covers them).  0 when M, N or K is 0.  splits = 0 asks for the
 * library's choice (below) and gives 0 where that choice is not to split.
 * GEMM_ERR_DIM for a negative size, GEMM_ERR_RANGE for a size >= 2^31 or
 * splits outside 0 .. 64.  No GPU call.
 *
 * gemm_run_splitk -- gemm_run_ex with K cut into pieces computed by different
 * workgroups (the work-splitting half of the stream-K scheduling in "The
 * Asynchronous Kernel: Tensor Cores & TMA", section "Keeping the line busy"),
 * for outputs with too few 256 x 256 tiles to occupy the GPU when K is long.
 * A first kernel computes, for every (output tile, piece), that piece's fp32
 * partial product into the workspace; a second kernel on the same stream adds
 * each element's partials in piece order (the result does not depend on
 * which workgroup finished first: repeated calls give the same bits),
 * applies act(alpha * sum + beta * C + bias[j]) in fp32 as gemm_run_ex does
 * and rounds once to the output type.  The k order differs from gemm_run's,
 * so results agree with it within the accumulation bound, not bit for bit
 * (with splits = 1 they are gemm_run_instance_ex's on the 256 x 256 instance,
 * bit for bit).
 *
 *   splits           requested pieces of K, 1 .. 64, or 0 for the library's
 *                    choice: split only when fewer than 128 tiles of 128 x 128
 *                    cover the output (more than half the GPU idle even on
 *                    the k-split kernel) and K >= 4096, into
 *                    min(ceil(192 / tiles of 256 x 256), K / 1024, 64) pieces;
 *                    otherwise run unsplit, exactly as gemm_run_ex (no
 *                    workspace used).  GEMM_ERR_RANGE outside 0 .. 64.
 *   workspace        device pointer, 256-byte aligned, at least
 *                    gemm_splitk_workspace_size(M, N, K, splits) bytes, on
 *                    the current device, owned by the caller; no initial
 *                    contents are needed.  It must not overlap A, B, C or the
 *                    bias (GEMM_ERR_ALIAS).  Calls that may run at the same
 *                    time need different workspaces.
 *   workspace_bytes  its size in bytes.
 *
 * Every dtype (the 8-bit inputs on their 256 x 256 tile with 128-deep
 * slices).  Other arguments, ownership and status codes as gemm_run_ex, plus
 * GEMM_ERR_WORKSPACE; GEMM_ERR_INSTANCE when the 256 x 256 kernels cannot run
 * the shape (row-major B with N % 8 != 0 -- N % 16 for 8-bit inputs -- and a
 * partial tile, or leading dimensions too large for their 32-bit offsets).  K == 0 needs no workspace
 * and runs as gemm_run_ex.  No allocation, no host synchronisation.
 */
int64_t gemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K, int splits);

int gemm_run_splitk(int64_t M, int64_t N, int64_t K, int dtype, int b_layout,
                    const void* A, int64_t lda, const void* B, int64_t ldb,
                    void* C, int64_t ldc, float alpha, float beta,
                    const float* bias, int relu, int splits, void* workspace,
                    int64_t workspace_bytes, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* gemm_strerror(int status);

/*
 * Kernel instances.  Each instance is one compiled kernel configuration; all
 * compute the same function.  Four families: "dl_*" (the waves of a
 * workgroup split its output tile; instances of this family give identical
 * bits), "pk_*" (the dl kernel's tiles taken from per-XCD queues by one
 * persistent workgroup per CU; gemm_run_ws only; bits identical to "dl_*"),
 * "ks_*" (the four waves split K over a 128x128 tile and their partial
 * sums are added in a fixed order, so repeated calls give identical bits; the
 * rounding differs from the dl family within the accuracy bound), and
 * "dl8_*" (the dl kernel for 8-bit inputs, which run only there; identical
 * bits within the family).  gemm_run picks one from the dtype, the shape, the
 * alignment, K and the number of output tiles.
 *
 * gemm_select_instance returns the id gemm_run would use for these arguments
 * (pointers are only inspected for alignment, never dereferenced; no GPU call
 * is made), or a negative GEMM_ERR_* code for arguments gemm_run rejects.
 * For no-op sizes (M == 0, N == 0 or K == 0) it returns GEMM_OK.
 */
int gemm_select_instance(int64_t M, int64_t N, int64_t K, int dtype,
                         const void* A, int64_t lda, const void* B, int64_t ldb,
                         const void* C, int64_t ldc);

/* gemm_select_instance for the arguments of gemm_run_ex (bias is inspected
 * for alignment and overlap only).  K == 0 with a general epilogue selects an
 * instance too: it evaluates act(beta*C + bias). */
int gemm_select_instance_ex(int64_t M, int64_t N, int64_t K, int dtype, int b_layout,
                            const void* A, int64_t lda, const void* B, int64_t ldb,
                            const void* C, int64_t ldc, float alpha, float beta,
                            const float* bias, int relu);

/* gemm_select_instance_ex for the arguments of gemm_run_ws (the workspace
 * is inspected for size, alignment and overlap only; the current device's
 * compute-unit count is queried). */
int gemm_select_instance_ws(int64_t M, int64_t N, int64_t K, int dtype, int b_layout,
                            const void* A, int64_t lda, const void* B, int64_t ldb,
                            const void* C, int64_t ldc, float alpha, float beta,
                            const float* bias, int relu, const void* workspace,
                            int64_t workspace_bytes);

/* Number of instance ids (0 .. gemm_num_instances()-1). */
int gemm_num_instances(void);

/* Static name of an instance id ("?" for an unknown id). */
const char* gemm_instance_name(int instance);

/*
 * gemm_run_instance -- gemm_run with the instance forced (for sweeps and for
 * the tests that require instances differing only in data movement or tile
 * order to agree bit for bit).  Same arguments, ownership and status codes as
 * gemm_run, plus GEMM_ERR_INSTANCE when `instance` is unknown or cannot
 * handle the shape or alignment.
 */
int gemm_run_instance(int instance, int64_t M, int64_t N, int64_t K, int dtype,
                      const void* A, int64_t lda, const void* B, int64_t ldb,
                      void* C, int64_t ldc, void* stream);

/* gemm_run_ws with the instance forced; the persistent "pk_*" instances run
 * only here (they need the workspace), on any shape their edge mode takes. */
int gemm_run_instance_ws(int instance, int64_t M, int64_t N, int64_t K, int dtype,
                         int b_layout, const void* A, int64_t lda, const void* B,
                         int64_t ldb, void* C, int64_t ldc, float alpha, float beta,
                         const float* bias, int relu, void* workspace,
                         int64_t workspace_bytes, void* stream);

/* gemm_run_ex with the instance forced; GEMM_ERR_INSTANCE as gemm_run_instance
 * (the prefetch-distance-1 instances run only the plain row-major form). */
int gemm_run_instance_ex(int instance, int64_t M, int64_t N, int64_t K, int dtype,
                         int b_layout, const void* A, int64_t lda, const void* B,
                         int64_t ldb, void* C, int64_t ldc, float alpha, float beta,
                         const float* bias, int relu, void* stream);

/*
 * gemm_tile_order -- host evaluation of an instance's workgroup-to-tile map
 * (the grouped CTA order of the Ada write-up, its table of DRAM bytes read per
 * CTA order at 4096^3 and 8192^3, applied per XCD).  For workgroup ids 0 .. count-1 of a launch
 * on an M x N output it writes the output tile row tm[w] and column tn[w].
 * Returns the number of workgroups of that launch, or a negative GEMM_ERR_*
 * code.  With tm == NULL or tn == NULL nothing is written.  No GPU call is
 * made.
 */
int64_t gemm_tile_order(int instance, int64_t M, int64_t N,
                        int32_t* tm, int32_t* tn, int64_t count);

#ifdef __cplusplus
}
#endif

#endif /* DHPT_GEMM_H */
