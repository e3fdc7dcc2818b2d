// gemm_instances.hip -- the instance table of the direct-to-LDS kernel family,
// what each instance can run, its launch, and the K == 0 fill.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_internal.h"

namespace dhpt {

// Every instance walks the output tiles in the XCD-aware grouped order of
// tile_coords with groups of 4 tile-rows: the 32 tiles an XCD runs at once
// cover 4 tile-rows x 8 tile-columns (12 panels, the minimum for 32 tiles,
// as 8 x 4 would be), and at 8192^3 each XCD keeps the same 4 A row-panels
// for the whole launch while all eight walk the same B column-panels
// together (measured: +2.4% at 8192^3, +1.5% at 4096^3 over groups of 8).
// New instances go at the end: the ids are part of the introspection
// interface.
const InstanceInfo kInstances[] = {
    {"dl_256x256x64_fd2", 256, 2, EDGE_NONE, 4, KIND_DL},
    {"dl_256x256x64_fd2_clamp", 256, 2, EDGE_CLAMP, 4, KIND_DL},
    {"dl_256x256x64_masked", 256, 2, EDGE_MASKED, 4, KIND_DL},
    {"dl_128x128x64_fd2", 128, 2, EDGE_NONE, 4, KIND_DL},
    {"dl_128x128x64_fd2_clamp", 128, 2, EDGE_CLAMP, 4, KIND_DL},
    {"dl_128x128x64_masked", 128, 2, EDGE_MASKED, 4, KIND_DL},
    {"dl_256x256x64_fd1", 256, 1, EDGE_NONE, 4, KIND_DL},
    {"dl_256x256x64_fd1_clamp", 256, 1, EDGE_CLAMP, 4, KIND_DL},
    {"dl_128x128x64_fd1", 128, 1, EDGE_NONE, 4, KIND_DL},
    {"dl_128x128x64_fd1_clamp", 128, 1, EDGE_CLAMP, 4, KIND_DL},
    {"ks_128x128x64", 128, 2, EDGE_NONE, 4, KIND_KS},
    {"ks_128x128x64_clamp", 128, 2, EDGE_CLAMP, 4, KIND_KS},
    {"dl_64x64x64_fd2", 64, 2, EDGE_NONE, 4, KIND_DL},
    {"dl_64x64x64_fd2_clamp", 64, 2, EDGE_CLAMP, 4, KIND_DL},
    // 8-bit float inputs: 128-deep slices, fragment prefetch one 64-deep k-step
    {"dl8_256x256x128", 256, 1, EDGE_NONE, 4, KIND_DL, 1},
    {"dl8_256x256x128_clamp", 256, 1, EDGE_CLAMP, 4, KIND_DL, 1},
    {"dl8_128x128x128", 128, 1, EDGE_NONE, 4, KIND_DL, 1},
    {"dl8_128x128x128_clamp", 128, 1, EDGE_CLAMP, 4, KIND_DL, 1},
    {"dl8_64x64x128", 64, 1, EDGE_NONE, 4, KIND_DL, 1},
    {"dl8_64x64x128_clamp", 64, 1, EDGE_CLAMP, 4, KIND_DL, 1},
    {"dl8_256x256x128_masked", 256, 1, EDGE_MASKED, 4, KIND_DL, 1},
    {"dl8_128x128x128_masked", 128, 1, EDGE_MASKED, 4, KIND_DL, 1},
    // persistent 256x256 kernels: tiles from per-XCD atomic queues in the
    // caller's workspace (gemm_run_ws)
    {"pk_256x256x64", 256, 2, EDGE_NONE, 4, KIND_PK},
    {"pk_256x256x64_clamp", 256, 2, EDGE_CLAMP, 4, KIND_PK},
    // ping-pong: two groups of four waves alternating multiplies and data
    // movement (whole 256x256 tiles); `fd` holds the k-steps per phase
    // (half a slice, or a whole slice)
    {"pp_256x256x64", 256, 2, EDGE_NONE, 4, KIND_PP},
    {"pp_256x256x64_ph4", 256, 4, EDGE_NONE, 4, KIND_PP},
};
const int kNumInstances = sizeof(kInstances) / sizeof(kInstances[0]);

// The asynchronous-copy kernels (whole-tile and clamped modes) address each
// lane's 16 bytes as a 32-bit byte offset from a per-tile base: at most
// tile - 1 rows of A (or of column-major B) plus a 128-byte slice, or one
// slice's 128 / esz rows of row-major B plus a tile width.  The offsets are
// kept below 2^31, where a signed and an unsigned reading of the offset
// agree.  Problems beyond that (leading dimensions of millions of elements)
// take the masked kernels, which fill through VGPRs with 64-bit addresses.
static bool copy_offsets_fit(const Problem& p, int tile, int esz) {
    const uint64_t lim = 0x7FFFFFFFull;
    const uint64_t a = (uint64_t)(tile - 1) * (uint64_t)p.lda * esz + 128;
    const uint64_t b = p.transB ? (uint64_t)(tile - 1) * (uint64_t)p.ldb * esz + 128
                                : (uint64_t)128 * (uint64_t)p.ldb + (uint64_t)tile * esz;
    return a <= lim && b <= lim;
}

// The clamped-edge kernels store edge tiles through a buffer descriptor over
// the tile's first element of C, with 32-bit byte offsets below 2^31: at most
// tile - 1 rows of ldc plus a tile width.  Larger leading dimensions of C take
// the masked kernels.
static bool c_offsets_fit(const Problem& p, int tile) {
    const uint64_t osz = dtype_out_f32(p.dtype) ? 4 : 2;
    return ((uint64_t)(tile - 1) * (uint64_t)p.ldc + (uint64_t)tile) * osz <= 0x7FFFFFFFull;
}

bool instance_supports(int id, const Problem& p) {
    if (id < 0 || id >= kNumInstances) return false;
    const InstanceInfo& in = kInstances[id];
    // one workgroup of 256 lanes per tile: the grid stays within 2^32 lanes
    const int64_t tiles = ((int64_t)(p.M + in.tile - 1) / in.tile) * ((p.N + in.tile - 1) / in.tile);
    if (tiles > (int64_t(1) << 24)) return false;
    if ((in.in8 != 0) != dtype_in8(p.dtype)) return false;                       // input width
    if (in.kind == KIND_PK && (p.sched == nullptr || p.workers <= 0)) return false;  // needs a workspace
    if (!in.in8 && in.kind == KIND_DL && in.fd == 1 && (p.transB || p.epi)) return false;   // plain row-major B only
    if (in.edge != EDGE_MASKED && !copy_offsets_fit(p, in.tile, in.in8 ? 1 : 2)) return false;
    switch (in.edge) {
    case EDGE_NONE:
        // whole tiles; C rows start on 64-byte boundaries, which the
        // non-temporal stores of these kernels need to write whole segments
        return p.M % in.tile == 0 && p.N % in.tile == 0 && p.K % (in.in8 ? 128 : 64) == 0 &&
               ((reinterpret_cast<uintptr_t>(p.C) | (uintptr_t)p.ldc * (dtype_out_f32(p.dtype) ? 4 : 2)) & 63) == 0;
    case EDGE_CLAMP: {
        const int chunk = in.in8 ? 16 : 8;                 // row-major B: whole 16-byte column chunks
        if (!c_offsets_fit(p, in.tile)) return false;
        return p.transB || (p.N % chunk == 0 && p.N >= chunk);
    }
    case EDGE_MASKED: return true;                       // any shape, any leading dimension
    default: return false;
    }
}

hipError_t launch_instance(int id, const Problem& p, hipStream_t s) {
    const InstanceInfo& in = kInstances[id];
    if (in.in8) {
        if (p.transB)
            return p.epi ? launch_dl_f8_tn_epi(in.tile, in.edge, p, in.group_m, s)
                         : launch_dl_f8_tn(in.tile, in.edge, p, in.group_m, s);
        return p.epi ? launch_dl_f8_nn_epi(in.tile, in.edge, p, in.group_m, s)
                     : launch_dl_f8_nn(in.tile, in.edge, p, in.group_m, s);
    }
    if (in.kind == KIND_KS)
        return p.epi ? launch_ks_epi(in.edge, p, in.group_m, s) : launch_ks(in.edge, p, in.group_m, s);
    if (in.kind == KIND_PP) return launch_pp(in.fd, p, in.group_m, s);
    if (in.kind == KIND_PK) {
        if (p.transB)
            return p.epi ? launch_pk_tn_epi(in.edge, p, in.group_m, s) : launch_pk_tn(in.edge, p, in.group_m, s);
        return p.epi ? launch_pk_nn_epi(in.edge, p, in.group_m, s) : launch_pk_nn(in.edge, p, in.group_m, s);
    }
    if (p.transB)
        return p.epi ? launch_dl_tn_epi(in.tile, in.fd, in.edge, p, in.group_m, s)
                     : launch_dl_tn(in.tile, in.fd, in.edge, p, in.group_m, s);
    return p.epi ? launch_dl_nn_epi(in.tile, in.fd, in.edge, p, in.group_m, s)
                 : launch_dl_nn(in.tile, in.fd, in.edge, p, in.group_m, s);
}

// C = 0 over the M x N region (K == 0 with the plain epilogue).
template <typename T>
__global__ __launch_bounds__(256) void zero_fill_kernel(T* C, int64_t ldc, int M, int N) {
    const int64_t total = (int64_t)M * N;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx / N, j = idx - i * N;
        C[i * ldc + j] = T(0);
    }
}

#ifdef DHPT_TIMELINE
static uint64_t* g_timeline = nullptr;
static int64_t g_timeline_waves = 0;

uint64_t* timeline_for(int64_t waves) { return waves <= g_timeline_waves ? g_timeline : nullptr; }
#endif

hipError_t launch_zero_fill(const Problem& p, hipStream_t s) {
    const int64_t total = (int64_t)p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    const dim3 grid((unsigned)blocks), block(256);
    if (dtype_out_f32(p.dtype))
        hipLaunchKernelGGL(zero_fill_kernel<float>, grid, block, 0, s, static_cast<float*>(p.C), p.ldc, p.M, p.N);
    else
        hipLaunchKernelGGL(zero_fill_kernel<uint16_t>, grid, block, 0, s, static_cast<uint16_t*>(p.C), p.ldc,
                           p.M, p.N);
    return hipGetLastError();
}

}  // namespace dhpt

#ifdef DHPT_TIMELINE
// Profiling builds only: register a device buffer of `waves` x 8 uint64
// words; every later launch whose waves fit records its per-wave timeline
// there (see tl_record).  A null buffer or waves <= 0 stops recording.
extern "C" int gemm_timeline_set(void* buf, int64_t waves) {
    dhpt::g_timeline = waves > 0 ? static_cast<uint64_t*>(buf) : nullptr;
    dhpt::g_timeline_waves = buf != nullptr && waves > 0 ? waves : 0;
    return 0;
}
#endif
