// gemm_internal.h -- shared between the C-ABI layer (gemm_api.cpp), the
// instance table (gemm_instances.hip) and the kernel instantiation units
// (gemm_dl_*.hip).  Not installed; callers use include/gemm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dhpt {

// One GEMM call after validation.  Sizes fit in int32 (checked by the API).
struct Problem {
    int M, N, K;
    int dtype;                 // gemm_dtype_t
    // Input bit patterns: 2-byte elements (fp16, bf16) or 1-byte elements
    // (8-bit floats); leading dimensions in elements.
    const uint16_t* A; int64_t lda;
    const uint16_t* B; int64_t ldb;
    void* C; int64_t ldc;
    bool transB;               // B stored column-major: B(k, j) at B[j*ldb + k]
    bool epi;                  // general epilogue (anything but alpha 1, beta 0, no bias, no ReLU)
    float alpha, beta;
    const float* bias;         // N fp32 values or null
    int relu;
    // Persistent kernels only: the zeroed scheduler words of the caller's
    // workspace (null without a workspace) and the number of workgroups to
    // launch (the device's compute units).
    uint32_t* sched;
    int workers;
};

// dtype facts shared by the API and the instance table.
inline bool dtype_in8(int dtype) { return dtype >= 4 && dtype <= 9; }           // 8-bit float inputs
inline bool dtype_out_f32(int dtype) { return dtype == 0 || dtype == 2 || dtype == 4 || dtype == 7; }

// Edge handling of an instance (the EDGE modes of gemm_dl_kernel.h).
enum EdgeMode {
    EDGE_NONE = 0,             // M % tile, N % tile, K % 64 == 0 (K % 128 for 8-bit inputs)
    EDGE_CLAMP = 1,            // any M, K; N % 8 == 0 (16 for 8-bit) for row-major B, any N column-major
    EDGE_MASKED = 2,           // any shape
};

// Kernel families.
enum KernelKind {
    KIND_DL = 0,               // gemm_dl_kernel.h: waves split the output tile
    KIND_KS = 1,               // gemm_ks_kernel.h: waves split K, 128x128 tile, LDS reduction
    KIND_PK = 2,               // gemm_dl_kernel.h, persistent: one workgroup per CU, tiles from
                               // per-XCD atomic queues (needs the workspace of gemm_run_ws)
    KIND_PP = 3,               // gemm_pp_kernel.h: 8 waves in two groups taking turns (ping-pong)
};

// Bytes of workspace the persistent kernels use (their scheduler words).
constexpr int64_t kWorkspaceBytes = 4096;

// One compiled kernel configuration.  The instances of one kind compute the
// same function with the same per-element operation order; the two kinds
// differ in the order the k-steps are summed.
struct InstanceInfo {
    const char* name;
    int tile;                  // square workgroup tile: 256 or 128 (k-slice 64)
    int fd;                    // fragment prefetch distance in k-steps (KIND_DL): 1 or 2;
                               // KIND_PP: k-steps per phase (2 or 4)
    int edge;                  // EdgeMode
    int group_m;               // tile-rows per group of the visit order
    int kind;                  // KernelKind
    int in8;                   // 1: 8-bit float inputs only; 0: 16-bit inputs only
};

extern const InstanceInfo kInstances[];
extern const int kNumInstances;

// True when instance `id` can run problem `p`.
bool instance_supports(int id, const Problem& p);

hipError_t launch_instance(int id, const Problem& p, hipStream_t stream);

#ifdef DHPT_TIMELINE
// Profiling builds: the buffer registered by gemm_timeline_set when it holds
// `waves` records of 8 words, else null (no recording).
uint64_t* timeline_for(int64_t waves);
#endif
hipError_t launch_zero_fill(const Problem& p, hipStream_t stream);

// The instantiation units of gemm_dl_kernel.h: row-major / column-major B,
// plain / general epilogue.  Only launch_dl_nn has fd == 1 kernels.
hipError_t launch_dl_nn(int tile, int fd, int edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_dl_nn_epi(int tile, int fd, int edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_dl_tn(int tile, int fd, int edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_dl_tn_epi(int tile, int fd, int edge, const Problem& p, int group_m, hipStream_t stream);
// The 8-bit-input units of gemm_dl_kernel.h (fd 1): column-major / row-major B,
// plain / general epilogue.
hipError_t launch_dl_f8_tn(int tile, int edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_dl_f8_tn_epi(int tile, int edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_dl_f8_nn(int tile, int edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_dl_f8_nn_epi(int tile, int edge, const Problem& p, int group_m, hipStream_t stream);
// The instantiation units of gemm_ks_kernel.h: plain / general epilogue (both B layouts).
hipError_t launch_ks(int edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_ks_epi(int edge, const Problem& p, int group_m, hipStream_t stream);
// The persistent 256x256 kernels (16-bit inputs): row-major / column-major B,
// plain / general epilogue.
hipError_t launch_pk_nn(int edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_pk_nn_epi(int edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_pk_tn(int edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_pk_tn_epi(int edge, const Problem& p, int group_m, hipStream_t stream);
// The ping-pong 256x256 kernel (16-bit inputs, whole tiles, both B layouts),
// `ph` k-steps per phase (2 or 4).
hipError_t launch_pp(int ph, const Problem& p, int group_m, hipStream_t stream);
// Split-K across workgroups (gemm_sk.hip, 256x256 tiles): the pieces
// launched for `splits` requested and their length Kc (a multiple of `gran`,
// the slice depth: 64 for 16-bit inputs, 128 for 8-bit ones), and the two
// launches (partial tiles into `ws`, then their sum and the epilogue into C);
// `edge` is EDGE_NONE or EDGE_CLAMP.
int splitk_pieces(int K, int splits, int gran, int* Kc);
hipError_t launch_splitk(const Problem& p, int splits, int edge, float* ws, int group_m, hipStream_t stream);

// Workgroup id -> output tile (tm, tn), in two steps, both bijections of
// [0, tilesM*tilesN).
//
// Step 1, XCD-aware remap (xcd_logical): MI355X deals consecutive workgroup
// ids round-robin over its 8 XCDs, each with its own L2.  Workgroup w (on
// XCD w % 8) is given logical id L so that XCD x owns one contiguous range of
// logical ids, [xcd_first(x), xcd_first(x + 1)); tiles that share an L2 are
// then neighbours in the visit order below.
//
// Step 2, grouped order (grouped_tile): logical ids walk `group_m` tile-rows
// at a time, down the column of a group before moving right, so the tiles in
// flight share a few A row-panels and B column-panels (the grouped CTA
// rasterization of the Ada tensor-core GEMM write-up, its section on the
// 8192^3 slowdown and the DRAM bytes each CTA order reads; and the
// 4x2-block example of "The Asynchronous Kernel: Tensor Cores & TMA",
// section "Scheduling is geometry").
__host__ __device__ inline int xcd_first(int x, int T) {
    const int q = T / 8, r = T % 8;
    return x * q + (x < r ? x : r);
}

__host__ __device__ inline int xcd_logical(int w, int T) { return xcd_first(w % 8, T) + w / 8; }

__host__ __device__ inline void grouped_tile(int L, int tilesM, int tilesN, int group_m, int* tm, int* tn) {
    const int per_group = group_m * tilesN;
    const int g = L / per_group;
    const int first_m = g * group_m;
    const int rows_left = tilesM - first_m;
    const int gsz = rows_left < group_m ? rows_left : group_m;
    const int within = L - g * per_group;
    *tm = first_m + within % gsz;
    *tn = within / gsz;
}

__host__ __device__ inline void tile_coords(int w, int tilesM, int tilesN, int group_m, int* tm, int* tn) {
    grouped_tile(xcd_logical(w, tilesM * tilesN), tilesM, tilesN, group_m, tm, tn);
}

}  // namespace dhpt
