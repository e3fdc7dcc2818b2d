// gemm_api.cpp -- the C ABI declared in include/gemm.h: argument validation,
// instance selection and the launch on the caller's stream.  No allocation,
// no host synchronisation, no per-call state (only per-device caches of the
// compute-unit count and of the static scratch's address).
#include "gemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gemm_internal.h"

namespace {

using dhpt::Problem;

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxLd = int64_t(1) << 40;
constexpr int64_t kMaxExtent = int64_t(1) << 47;   // elements spanned by one operand
constexpr int kMaxSplits = 64;                        // gemm_run_splitk: pieces of K

int out_elem_size(int dtype) { return dhpt::dtype_out_f32(dtype) ? 4 : 2; }
int in_elem_size(int dtype) { return dhpt::dtype_in8(dtype) ? 1 : 2; }

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

// Byte extent [begin, end) of a rows x cols row-major matrix with leading dim ld.
void extent(const void* p, int64_t rows, int64_t cols, int64_t ld, int esz, uintptr_t* b, uintptr_t* e) {
    *b = reinterpret_cast<uintptr_t>(p);
    *e = *b + (uintptr_t)(((rows - 1) * ld + cols) * esz);
}

// The epilogue and layout arguments of gemm_run_ex (gemm_run: the defaults),
// and the workspace of gemm_run_ws.
struct Extra {
    int b_layout = GEMM_B_ROW_MAJOR;
    float alpha = 1.0f, beta = 0.0f;
    const float* bias = nullptr;
    int relu = 0;
    void* ws = nullptr;
    int64_t ws_bytes = 0;
};

// Compute units of the current device (the persistent kernels launch one
// workgroup per CU), queried once per device and kept: a property of the
// device, not of any call.
int device_cus() {
    static std::atomic<int> cached[64];        // zero until the first call on a device (any thread)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Validate; on success fill `p` and return GEMM_OK (and *noop for empty output).
int validate(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
             const void* B, int64_t ldb, const void* C, int64_t ldc, const Extra& x, Problem* p,
             bool* noop) {
    *noop = false;
    if (dtype < GEMM_F16_F32 || dtype > GEMM_E5M2_BF16) return GEMM_ERR_DTYPE;
    if (x.b_layout != GEMM_B_ROW_MAJOR && x.b_layout != GEMM_B_COL_MAJOR) return GEMM_ERR_LAYOUT;
    const bool tb = x.b_layout == GEMM_B_COL_MAJOR;
    const int64_t b_rows = tb ? N : K, b_cols = tb ? K : N;      // B as stored, row-major
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_DIM;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMM_ERR_RANGE;
    if (lda < 0 || ldb < 0 || ldc < 0) return GEMM_ERR_LD;
    if (lda > kMaxLd || ldb > kMaxLd || ldc > kMaxLd) return GEMM_ERR_RANGE;
    if (lda < K || ldb < b_cols || ldc < N) return GEMM_ERR_LD;
    // byte extents stay far below 2^63, and the tile grid fits a 32-bit launch
    if ((M > 1 && lda > kMaxExtent / (M - 1)) || (b_rows > 1 && ldb > kMaxExtent / (b_rows - 1)) ||
        (M > 1 && ldc > kMaxExtent / (M - 1)))
        return GEMM_ERR_RANGE;
    if (((M + 127) / 128) * ((N + 127) / 128) > kMaxDim) return GEMM_ERR_RANGE;
    if (M == 0 || N == 0) { *noop = true; return GEMM_OK; }
    if (C == nullptr) return GEMM_ERR_NULL;
    if (K > 0 && (A == nullptr || B == nullptr)) return GEMM_ERR_NULL;
    const int osz = out_elem_size(dtype), isz = in_elem_size(dtype);
    if (reinterpret_cast<uintptr_t>(C) % osz != 0) return GEMM_ERR_ALIGN;
    if (K > 0 && (reinterpret_cast<uintptr_t>(A) % isz != 0 || reinterpret_cast<uintptr_t>(B) % isz != 0))
        return GEMM_ERR_ALIGN;
    if (x.bias != nullptr && reinterpret_cast<uintptr_t>(x.bias) % 4 != 0) return GEMM_ERR_ALIGN;
    uintptr_t c0, c1;
    extent(C, M, N, ldc, osz, &c0, &c1);
    if (K > 0) {
        uintptr_t a0, a1, b0, b1;
        extent(A, M, K, lda, isz, &a0, &a1);
        extent(B, b_rows, b_cols, ldb, isz, &b0, &b1);
        if (overlaps(c0, c1, a0, a1) || overlaps(c0, c1, b0, b1)) return GEMM_ERR_ALIAS;
    }
    if (x.bias != nullptr) {
        const uintptr_t z0 = reinterpret_cast<uintptr_t>(x.bias), z1 = z0 + (uintptr_t)(4 * N);
        if (overlaps(c0, c1, z0, z1)) return GEMM_ERR_ALIAS;
    }
    if (x.ws != nullptr) {
        if (x.ws_bytes < dhpt::kWorkspaceBytes || reinterpret_cast<uintptr_t>(x.ws) % 256 != 0)
            return GEMM_ERR_WORKSPACE;
        const uintptr_t w0 = reinterpret_cast<uintptr_t>(x.ws), w1 = w0 + (uintptr_t)dhpt::kWorkspaceBytes;
        if (overlaps(c0, c1, w0, w1)) return GEMM_ERR_ALIAS;
        if (K > 0) {
            uintptr_t a0, a1, b0, b1;
            extent(A, M, K, lda, isz, &a0, &a1);
            extent(B, b_rows, b_cols, ldb, isz, &b0, &b1);
            if (overlaps(w0, w1, a0, a1) || overlaps(w0, w1, b0, b1)) return GEMM_ERR_ALIAS;
        }
        if (x.bias != nullptr) {
            const uintptr_t z0 = reinterpret_cast<uintptr_t>(x.bias), z1 = z0 + (uintptr_t)(4 * N);
            if (overlaps(w0, w1, z0, z1)) return GEMM_ERR_ALIAS;
        }
    }
    p->M = (int)M; p->N = (int)N; p->K = (int)K; p->dtype = dtype;
    p->A = static_cast<const uint16_t*>(A); p->lda = lda;
    p->B = static_cast<const uint16_t*>(B); p->ldb = ldb;
    p->C = const_cast<void*>(C); p->ldc = ldc;
    p->transB = tb;
    p->alpha = x.alpha; p->beta = x.beta; p->bias = x.bias; p->relu = x.relu != 0;
    p->epi = !(x.alpha == 1.0f && x.beta == 0.0f && x.bias == nullptr && x.relu == 0);
    p->sched = static_cast<uint32_t*>(x.ws);
    p->workers = 0;
    return GEMM_OK;
}

int64_t tiles_for(int tile, int64_t M, int64_t N) { return ((M + tile - 1) / tile) * ((N + tile - 1) / tile); }

// Large (256x256) tiles when they still give at least half a wave over the
// 256 CUs.  Otherwise:
//  * K >= 2048 and at least 64 tiles of 128x128: the k-split kernel (each
//    wave accumulates the whole 128x128 tile over a quarter of the k-steps:
//    fewer LDS bytes per MFMA, paid for by a reduction through LDS);
//  * fewer than 128 tiles of 128x128 and K <= 2048: 64x64 tiles, four times
//    the workgroups (small problems are bound by latency, not by bytes);
//  * else 128x128 tiles, each wave a quarter of the tile.
// Within a family, the first instance that supports the problem: whole
// tiles, then clamped edges (any M and K; N a multiple of 8 for row-major
// B), then the fully masked fallback (128x128).
//
// 8-bit inputs: 256x256 tiles when they give at least half a wave, else
// 128x128 tiles when those give at least half a wave, else 64x64; whole
// tiles, then clamped edges (every shape with column-major B, N % 16 == 0
// with row-major B), then the masked fallback (row-major B, any N).
//
// With a workspace (gemm_run_ws), 16-bit inputs with at least two 256x256
// tiles per compute unit run on the persistent kernel: the tail of the
// launch is then balanced across XCDs that hold different clocks (with one
// tile per CU or fewer there is nothing to rebalance).
int choose_instance(const Problem& p) {
    if (p.sched != nullptr && p.workers > 0 && !dhpt::dtype_in8(p.dtype) &&
        tiles_for(256, p.M, p.N) >= 2 * (int64_t)p.workers) {
        static const int pk_order[] = {22, 23};
        for (int k = 0; k < 2; ++k)
            if (dhpt::instance_supports(pk_order[k], p)) return pk_order[k];
    }
    if (dhpt::dtype_in8(p.dtype)) {
        static const int big8[] = {14, 15, 20}, mid8[] = {16, 17, 21}, small8[] = {18, 19, 21};
        const int* o = tiles_for(256, p.M, p.N) >= 128 ? big8 : tiles_for(128, p.M, p.N) >= 128 ? mid8 : small8;
        for (int k = 0; k < 3; ++k)
            if (dhpt::instance_supports(o[k], p)) return o[k];
        return o[2];
    }
    static const int big_order[] = {0, 1, 2};
    static const int mid_order[] = {3, 4, 5};
    static const int ks_order[] = {10, 11, 5};
    static const int small_order[] = {12, 13, 5};
    const int64_t t128 = tiles_for(128, p.M, p.N);
    const int* order = tiles_for(256, p.M, p.N) >= 128      ? big_order
                       : (p.K >= 2048 && t128 >= 64)        ? ks_order
                       : (t128 < 128 && p.K <= 2048)        ? small_order
                                                            : mid_order;
    for (int k = 0; k < 3; ++k)
        if (dhpt::instance_supports(order[k], p)) return order[k];
    return order[2];
}

int enqueue(int id, const Problem& p, hipStream_t s) {
    hipError_t err = hipGetLastError();   // clear a stale error so it is not blamed on this launch
    (void)err;
    err = dhpt::launch_instance(id, p, s);
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

// K == 0: the product is the zero matrix.  The plain form writes zeros; the
// general form still has act(beta*C + bias) to evaluate, which the kernels do
// with an empty k loop.
int run_validated(int instance, const Problem& p, hipStream_t s) {
    if (p.K == 0 && !p.epi) {
        (void)hipGetLastError();
        return dhpt::launch_zero_fill(p, s) == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
    }
    if (instance < 0) instance = choose_instance(p);
    else if (!dhpt::instance_supports(instance, p)) return GEMM_ERR_INSTANCE;
    return enqueue(instance, p, s);
}

int run_any(int instance, int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
            const void* B, int64_t ldb, void* C, int64_t ldc, const Extra& x, void* stream) {
    Problem p;
    bool noop;
    int st = validate(M, N, K, dtype, A, lda, B, ldb, C, ldc, x, &p, &noop);
    if (st != GEMM_OK || noop) return st;
    if (p.sched != nullptr) p.workers = device_cus();
    return run_validated(instance, p, static_cast<hipStream_t>(stream));
}

int select_any(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda, const void* B,
               int64_t ldb, const void* C, int64_t ldc, const Extra& x) {
    Problem p;
    bool noop;
    int st = validate(M, N, K, dtype, A, lda, B, ldb, C, ldc, x, &p, &noop);
    if (st != GEMM_OK) return st;
    if (p.sched != nullptr) p.workers = device_cus();
    if (noop || (K == 0 && !p.epi)) return GEMM_OK;
    return choose_instance(p);
}

Extra extra(int b_layout, float alpha, float beta, const float* bias, int relu, void* ws = nullptr,
            int64_t ws_bytes = 0) {
    Extra x;
    x.b_layout = b_layout; x.alpha = alpha; x.beta = beta; x.bias = bias; x.relu = relu;
    x.ws = ws; x.ws_bytes = ws_bytes;
    return x;
}

// ---------------------------------------------------------------------------
// The allocation-free entry point's scratch (gemm_run_noalloc): the
// persistent kernels' scheduler words in a file-scope device array instead of
// a caller's workspace.  Each device that runs the library holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device address: the address is taken once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// passed to kernels.
constexpr int64_t kScratchBytes = 4096;
static_assert(dhpt::kWorkspaceBytes <= kScratchBytes, "the static scratch holds the persistent kernels' words");
__device__ __attribute__((aligned(256))) static uint32_t scratch[kScratchBytes / 4];

// Zero n words of the scratch (a kernel rather than hipMemsetAsync, so that
// the call can be captured in a HIP graph and replayed).
__global__ void scratch_clear_kernel(uint32_t* p, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;

// The device address of this device's scratch, looked up on the first call
// on the device and kept (each device has its own copy of the array at its
// own address).
int device_scratch(void** out) {
    static std::atomic<void*> ptrs[kMaxDevices];   // threads racing on a first call store the same address
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GEMM_ERR_LAUNCH;
    void* ptr = ptrs[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return GEMM_ERR_LAUNCH;
        }
        ptrs[dev].store(ptr, std::memory_order_relaxed);
    }
    *out = ptr;
    return GEMM_OK;
}

}  // namespace

extern "C" {

int gemm_run(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
             const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    return run_any(-1, M, N, K, dtype, A, lda, B, ldb, C, ldc, Extra(), stream);
}

int gemm_run_ex(int64_t M, int64_t N, int64_t K, int dtype, int b_layout, const void* A, int64_t lda,
                const void* B, int64_t ldb, void* C, int64_t ldc, float alpha, float beta,
                const float* bias, int relu, void* stream) {
    return run_any(-1, M, N, K, dtype, A, lda, B, ldb, C, ldc, extra(b_layout, alpha, beta, bias, relu),
                   stream);
}

int gemm_run_instance(int instance, int64_t M, int64_t N, int64_t K, int dtype, const void* A,
                      int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, void* stream) {
    if (instance < 0 || instance >= dhpt::kNumInstances) return GEMM_ERR_INSTANCE;
    return run_any(instance, M, N, K, dtype, A, lda, B, ldb, C, ldc, Extra(), stream);
}

int gemm_run_instance_ex(int instance, int64_t M, int64_t N, int64_t K, int dtype, int b_layout,
                         const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                         float alpha, float beta, const float* bias, int relu, void* stream) {
    if (instance < 0 || instance >= dhpt::kNumInstances) return GEMM_ERR_INSTANCE;
    return run_any(instance, M, N, K, dtype, A, lda, B, ldb, C, ldc,
                   extra(b_layout, alpha, beta, bias, relu), stream);
}

int gemm_select_instance(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int64_t lda,
                         const void* B, int64_t ldb, const void* C, int64_t ldc) {
    return select_any(M, N, K, dtype, A, lda, B, ldb, C, ldc, Extra());
}

int gemm_select_instance_ex(int64_t M, int64_t N, int64_t K, int dtype, int b_layout, const void* A,
                            int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc,
                            float alpha, float beta, const float* bias, int relu) {
    return select_any(M, N, K, dtype, A, lda, B, ldb, C, ldc, extra(b_layout, alpha, beta, bias, relu));
}

int64_t gemm_workspace_size(void) { return dhpt::kWorkspaceBytes; }

int gemm_run_ws(int64_t M, int64_t N, int64_t K, int dtype, int b_layout, const void* A, int64_t lda,
                const void* B, int64_t ldb, void* C, int64_t ldc, float alpha, float beta,
                const float* bias, int relu, void* workspace, int64_t workspace_bytes, void* stream) {
    if (workspace == nullptr) return GEMM_ERR_WORKSPACE;
    return run_any(-1, M, N, K, dtype, A, lda, B, ldb, C, ldc,
                   extra(b_layout, alpha, beta, bias, relu, workspace, workspace_bytes), stream);
}

int gemm_run_instance_ws(int instance, int64_t M, int64_t N, int64_t K, int dtype, int b_layout,
                         const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                         float alpha, float beta, const float* bias, int relu, void* workspace,
                         int64_t workspace_bytes, void* stream) {
    if (instance < 0 || instance >= dhpt::kNumInstances) return GEMM_ERR_INSTANCE;
    if (workspace == nullptr) return GEMM_ERR_WORKSPACE;
    return run_any(instance, M, N, K, dtype, A, lda, B, ldb, C, ldc,
                   extra(b_layout, alpha, beta, bias, relu, workspace, workspace_bytes), stream);
}

int gemm_select_instance_ws(int64_t M, int64_t N, int64_t K, int dtype, int b_layout, const void* A,
                            int64_t lda, const void* B, int64_t ldb, const void* C, int64_t ldc,
                            float alpha, float beta, const float* bias, int relu, const void* workspace,
                            int64_t workspace_bytes) {
    if (workspace == nullptr) return GEMM_ERR_WORKSPACE;
    return select_any(M, N, K, dtype, A, lda, B, ldb, C, ldc,
                      extra(b_layout, alpha, beta, bias, relu, const_cast<void*>(workspace), workspace_bytes));
}

int gemm_run_noalloc(int64_t M, int64_t N, int64_t K, int dtype, int b_layout, const void* A, int64_t lda,
                     const void* B, int64_t ldb, void* C, int64_t ldc, float alpha, float beta,
                     const float* bias, int relu, void* stream) {
    Problem p;
    bool noop;
    // validate first against a stand-in workspace address: the arguments,
    // not the scratch, decide whether the call is valid
    Extra x = extra(b_layout, alpha, beta, bias, relu);
    int st = validate(M, N, K, dtype, A, lda, B, ldb, C, ldc, x, &p, &noop);
    if (st != GEMM_OK || noop) return st;
    void* scratch_ptr = nullptr;
    st = device_scratch(&scratch_ptr);
    if (st != GEMM_OK) return st;
    x.ws = scratch_ptr;
    x.ws_bytes = kScratchBytes;
    st = validate(M, N, K, dtype, A, lda, B, ldb, C, ldc, x, &p, &noop);
    if (st != GEMM_OK) return st;
    p.workers = device_cus();
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.K == 0 && !p.epi) return run_validated(-1, p, s);
    const int inst = choose_instance(p);
    if (dhpt::kInstances[inst].kind == dhpt::KIND_PK) {
        if (dhpt::kWorkspaceBytes > kScratchBytes) return GEMM_ERR_WORKSPACE;
        // every call on this device shares the array: clear the scheduler
        // words (a fill kernel, not a memset, so that a captured graph
        // replays it correctly)
        (void)hipGetLastError();
        hipLaunchKernelGGL(scratch_clear_kernel, dim3(1), dim3(256), 0, s, static_cast<uint32_t*>(scratch_ptr),
                           (int)(dhpt::kWorkspaceBytes / 4));
        if (hipGetLastError() != hipSuccess) return GEMM_ERR_LAUNCH;
    }
    return run_validated(inst, p, s);
}

// splits == 0 for gemm_run_splitk: split only where even 128x128 tiles leave
// more than half the compute units idle (fewer than 128 of them) and K is
// long (>= 4096), into enough pieces for about 192 workgroups (three
// quarters of the CUs: more pieces add partial-tile traffic faster than they
// add compute), but none shorter than 1024.  Fitted on a sweep of 2 .. 64
// pieces (one box, bf16 TFLOP/s, unsplit -> this rule -> best): 512^2 x 32768
// 57 -> 446 (32 pieces, the best); 1024^2 x 16384 390 -> 719 (12, the best);
// 768^2 x 16384 129 -> 512 (16, the best); 1024^2 x 8192 364 -> 516 (8, the
// best); 512^2 x 8192 58 -> 156 (8; 183 at 16); 256^2 x 65536 15 -> 201 (64,
// the best); and 1024 x 2048 x 8192, 128 tiles of 128^2, stays unsplit (699
// on the k-split kernel, 675 in 4 pieces).  1 means no split.
int splitk_auto(int64_t M, int64_t N, int64_t K) {
    if (tiles_for(128, M, N) >= 128 || K < 4096) return 1;
    const int64_t t256 = tiles_for(256, M, N);
    int64_t s = (192 + t256 - 1) / t256;
    if (s > K / 1024) s = K / 1024;
    if (s > kMaxSplits) s = kMaxSplits;
    return s < 1 ? 1 : (int)s;
}

int64_t gemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K, int splits) {
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_DIM;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim || splits < 0 || splits > kMaxSplits) return GEMM_ERR_RANGE;
    if (M == 0 || N == 0 || K == 0) return 0;
    if (splits == 0) {
        splits = splitk_auto(M, N, K);
        if (splits == 1) return 0;                      // runs unsplit: no workspace
    }
    int Kc = 0;
    // pieces of 64-multiple length: the 16-bit count, which bounds the 8-bit
    // one (pieces of 128-multiple length, never more of them)
    const int64_t pieces = dhpt::splitk_pieces((int)K, splits, 64, &Kc);
    return tiles_for(256, M, N) * pieces * 256 * 256 * 4;
}

int gemm_run_splitk(int64_t M, int64_t N, int64_t K, int dtype, int b_layout, const void* A, int64_t lda,
                    const void* B, int64_t ldb, void* C, int64_t ldc, float alpha, float beta,
                    const float* bias, int relu, int splits, void* workspace, int64_t workspace_bytes,
                    void* stream) {
    Problem p;
    bool noop;
    int st = validate(M, N, K, dtype, A, lda, B, ldb, C, ldc, extra(b_layout, alpha, beta, bias, relu), &p, &noop);
    if (st != GEMM_OK) return st;
    if (splits < 0 || splits > kMaxSplits) return GEMM_ERR_RANGE;
    if (noop) return GEMM_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.K == 0) return run_validated(-1, p, s);          // no product to split: act(beta*C + bias) or zeros
    if (splits == 0) {
        splits = splitk_auto(M, N, K);
        if (splits == 1) return run_validated(-1, p, s);  // not worth splitting: gemm_run_ex's kernels
    }
    const int64_t need = gemm_splitk_workspace_size(M, N, K, splits);
    if (workspace == nullptr || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
        return GEMM_ERR_WORKSPACE;
    const bool in8 = dhpt::dtype_in8(dtype);
    int Kc = 0;
    const int64_t pieces = dhpt::splitk_pieces(p.K, splits, in8 ? 128 : 64, &Kc);
    if (tiles_for(256, M, N) * pieces > (int64_t(1) << 24)) return GEMM_ERR_RANGE;
    {
        const bool tb = b_layout == GEMM_B_COL_MAJOR;
        const int osz = out_elem_size(dtype), isz = in_elem_size(dtype);
        uintptr_t c0, c1, a0, a1, b0, b1;
        extent(C, M, N, ldc, osz, &c0, &c1);
        extent(A, M, K, lda, isz, &a0, &a1);
        extent(B, tb ? N : K, tb ? K : N, ldb, isz, &b0, &b1);
        const uintptr_t w0 = reinterpret_cast<uintptr_t>(workspace), w1 = w0 + (uintptr_t)need;
        if (overlaps(w0, w1, c0, c1) || overlaps(w0, w1, a0, a1) || overlaps(w0, w1, b0, b1)) return GEMM_ERR_ALIAS;
        if (bias != nullptr) {
            const uintptr_t z0 = reinterpret_cast<uintptr_t>(bias), z1 = z0 + (uintptr_t)(4 * N);
            if (overlaps(w0, w1, z0, z1)) return GEMM_ERR_ALIAS;
        }
    }
    // The pieces run the 256x256 tile of instance 0 / 14 (whole tiles) or
    // 1 / 15 (clamped edges; 16-bit / 8-bit inputs) on sub-problems with the
    // same leading dimensions, so those instances' limits apply.
    const int whole_id = in8 ? 14 : 0, clamp_id = in8 ? 15 : 1;
    const bool whole = M % 256 == 0 && N % 256 == 0 && K % (in8 ? 128 : 64) == 0;
    int edge;
    if (whole && dhpt::instance_supports(whole_id, p)) edge = dhpt::EDGE_NONE;
    else if (dhpt::instance_supports(clamp_id, p)) edge = dhpt::EDGE_CLAMP;
    else return GEMM_ERR_INSTANCE;
    (void)hipGetLastError();
    const hipError_t err = dhpt::launch_splitk(p, splits, edge, static_cast<float*>(workspace),
                                               dhpt::kInstances[0].group_m, s);
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int gemm_num_instances(void) { return dhpt::kNumInstances; }

const char* gemm_instance_name(int instance) {
    if (instance < 0 || instance >= dhpt::kNumInstances) return "?";
    return dhpt::kInstances[instance].name;
}

int64_t gemm_tile_order(int instance, int64_t M, int64_t N, int32_t* tm, int32_t* tn, int64_t count) {
    if (instance < 0 || instance >= dhpt::kNumInstances) return GEMM_ERR_INSTANCE;
    if (M < 0 || N < 0) return GEMM_ERR_DIM;
    if (M > kMaxDim || N > kMaxDim) return GEMM_ERR_RANGE;
    const dhpt::InstanceInfo& in = dhpt::kInstances[instance];
    const int64_t T = tiles_for(in.tile, M, N);
    if (T > kMaxDim) return GEMM_ERR_RANGE;
    const int64_t tilesM = (M + in.tile - 1) / in.tile, tilesN = (N + in.tile - 1) / in.tile;
    if (tm != nullptr && tn != nullptr) {
        const int64_t n = count < T ? count : T;
        for (int64_t w = 0; w < n; ++w) {
            int a, b;
            dhpt::tile_coords((int)w, (int)tilesM, (int)tilesN, in.group_m, &a, &b);
            tm[w] = a;
            tn[w] = b;
        }
    }
    return T;
}

const char* gemm_strerror(int status) {
    switch (status) {
    case GEMM_OK: return "success";
    case GEMM_ERR_DIM: return "negative dimension";
    case GEMM_ERR_LD: return "leading dimension smaller than the row length (lda < K, ldb < N or ldc < N; "
                             "ldb < K for column-major B)";
    case GEMM_ERR_NULL: return "null pointer for a non-empty operand";
    case GEMM_ERR_DTYPE: return "unknown dtype";
    case GEMM_ERR_ALIAS: return "C overlaps A, B or the bias";
    case GEMM_ERR_RANGE: return "dimension or leading dimension out of the supported range";
    case GEMM_ERR_LAUNCH: return "kernel launch failed";
    case GEMM_ERR_ALIGN: return "pointer not aligned to its element size";
    case GEMM_ERR_INSTANCE: return "unknown instance, or instance cannot run this shape";
    case GEMM_ERR_LAYOUT: return "unknown B layout";
    case GEMM_ERR_WORKSPACE: return "workspace missing, smaller than gemm_workspace_size() or not 256-byte aligned";
    default: return "unknown status";
    }
}

}  // extern "C"
