// gemm_internal.h -- shared between the C-ABI layer (gemm_api.cpp) and the
// kernels (gemm_kernels.hip).  Not installed; callers use include/gemm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dhpt {

// One GEMM call after validation.  Sizes fit in int32 (checked by the API).
struct Problem {
    int M, N, K;
    int dtype;                 // gemm_dtype_t
    const uint16_t* A; int64_t lda;
    const uint16_t* B; int64_t ldb;
    void* C; int64_t ldc;
    bool vecA, vecB;           // 16-byte aligned base and leading dimension
};

// What an instance requires of the problem.
enum Requirement {
    REQ_ANY = 0,               // any shape, any alignment (element-masked edges)
    REQ_TILE_VEC = 1,          // M % bm, N % bn, K % bk == 0 and 16-byte aligned A, B rows
    REQ_TILE = 2,              // M % bm, N % bn, K % bk == 0 (any 2-byte alignment)
    REQ_N8 = 3,                // N % 8 == 0 and N >= 8 (clamped edges, zero-filled K tail)
};

// One compiled tile geometry.  Every instance computes the same function.
struct InstanceInfo {
    const char* name;
    int bm, bn, bk;            // workgroup tile
    bool edge;                 // handles partial tiles (masked stores)
    int group_m;               // tile-rows per group of the visit order
    int req;                   // Requirement
};

extern const InstanceInfo kInstances[];
extern const int kNumInstances;

// True when instance `id` can run problem `p` (shape multiple of its tile and
// vector-aligned operands, or an edge instance).
bool instance_supports(int id, const Problem& p);

hipError_t launch_instance(int id, const Problem& p, hipStream_t stream);

// The direct-to-LDS family (gemm_dl.hip): tile 256 or 128, fragment prefetch
// distance 1 or 2, edge handling on or off.
hipError_t launch_dl(int tile, int fd, bool edge, const Problem& p, int group_m, hipStream_t stream);
hipError_t launch_zero_fill(const Problem& p, hipStream_t stream);

// Workgroup id -> output tile (tm, tn).
//
// Step 1, XCD-aware remap: MI355X deals consecutive workgroup ids round-robin
// over its 8 XCDs, each with its own L2.  Workgroup w (on XCD w % 8) is given
// logical id L so that XCD x owns one contiguous range of logical ids; tiles
// that share an L2 are then neighbours in the visit order below.
//
// Step 2, grouped order: logical ids walk `group_m` tile-rows at a time, down
// the column of a group before moving right, so the tiles in flight share a
// few A row-panels and B column-panels (the grouped CTA rasterization of the
// Ada tensor-core GEMM write-up, section "This one wasn't in the plan" on the
// 8192^3 slowdown; and the 4x2-block example of "The Asynchronous Kernel:
// Tensor Cores & TMA", section "Scheduling is geometry").
//
// Both steps are bijections of [0, tilesM*tilesN).
__host__ __device__ inline void tile_coords(int w, int tilesM, int tilesN, int group_m,
                                            int* tm, int* tn) {
    const int T = tilesM * tilesN;
    const int q = T / 8, r = T % 8;
    const int x = w % 8, i = w / 8;
    const int L = x * q + (x < r ? x : r) + i;
    const int per_group = group_m * tilesN;
    const int g = L / per_group;
    const int first_m = g * group_m;
    const int rows_left = tilesM - first_m;
    const int gsz = rows_left < group_m ? rows_left : group_m;
    const int within = L - g * per_group;
    *tm = first_m + within % gsz;
    *tn = within / gsz;
}

}  // namespace dhpt
