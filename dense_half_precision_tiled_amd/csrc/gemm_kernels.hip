// gemm_kernels.hip -- gfx950 (MI355X, CDNA4) MFMA kernels for C = A.B.
//
// Row-major A [M,K] and B [K,N] in fp16 or bf16, fp32 accumulation, fp32 /
// fp16 / bf16 output.  One workgroup of 4 waves (256 lanes) owns a BM x BN
// output tile and streams K through LDS in BK = 64 slices.
//
// Per k-slice (the staging structure of the Ada tensor-core GEMM write-up,
// sections on cp.async stages and on the pipelined main loop of "GEMM From
// Naive CUDA to Tensor Cores", "Where asynchronous copies and TMA take over"):
//   * global -> registers: each lane loads 16-byte chunks of the next slice
//     while the MFMAs of the current slice run;
//   * registers -> LDS: A is written as it was read (k contiguous); B, which
//     is row-major (n contiguous) while the MFMA B operand wants 8 consecutive
//     k of one column per lane, is transposed in registers (8x8 or 4x8 blocks
//     of 16-bit values) and written k-contiguous;
//   * two LDS stages, one workgroup barrier per k-slice: the stage being
//     filled is the one every wave finished reading before the last barrier,
//     and the stage being read was filled before it (the RAW and WAR barriers
//     of "GEMM From Naive CUDA to Tensor Cores", "Turn global loads into
//     shared tiles", folded into one by double buffering);
//   * LDS layout: 128-byte rows (64 halves) of eight 16-byte chunks, chunk c of
//     row r stored at position c ^ (r & 7) (the XOR swizzle of "The Asynchronous
//     Kernel: Tensor Cores & TMA", section "The XOR that unties the banks"), so
//     the row-wise fragment reads of 8 consecutive rows hit 8 different
//     16-byte bank groups, and so do the transposed-B writes;
//   * LDS -> VGPR: one ds_read_b128 per 32x16 fragment of A or B^T;
//   * v_mfma_f32_32x32x16_{f16,bf16}: D(32x32, fp32) += A(32x16) * B(16x32).
// The epilogue converts the fp32 accumulators once and stores them, masked at
// the M and N edges (the predicated final store of "Turn global loads into
// shared tiles").
//
// Register layouts of v_mfma_f32_32x32x16 (lane l of 64, g = l / 32):
//   A operand: row l % 32, 8 values of k;  B operand: column l % 32, the same
//   8 values of k;  (both use k = 16*s + 8*g + 0..7 here: any assignment of k
//   to (g, element) is valid as long as A and B use the same one.)
//   D: element i (0..15) is row 8*(i/4) + 4*g + (i%4), column l % 32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_internal.h"

namespace dhpt {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum { IN_F16 = 0, IN_BF16 = 1 };
enum { OUT_F32 = 0, OUT_F16 = 1, OUT_BF16 = 2 };

template <int IN>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (IN == IN_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int OUT>
__device__ __forceinline__ void store_out(void* C, int64_t idx, float v) {
    if constexpr (OUT == OUT_F32)
        static_cast<float*>(C)[idx] = v;
    else if constexpr (OUT == OUT_F16)
        static_cast<_Float16*>(C)[idx] = (_Float16)v;     // v_cvt_f16_f32: RNE
    else
        static_cast<__bf16*>(C)[idx] = (__bf16)v;         // RNE
}

// Two 16-bit values, column j of rows x (low half) and y (high half).
__device__ __forceinline__ uint32_t pack_col(u32x4 x, u32x4 y, int j) {
    const uint32_t xv = x[j >> 1], yv = y[j >> 1];
    return (j & 1) ? ((xv >> 16) | (yv & 0xffff0000u)) : ((xv & 0xffffu) | (yv << 16));
}

// Masked 8-element load: row `p` (already offset to the row), columns
// c0 .. c0+7 of which only those < limit exist; missing ones read as zero.
__device__ __forceinline__ u32x4 load_chunk_masked(const uint16_t* p, int c0, int limit, bool vec) {
    if (vec && c0 + 8 <= limit) return *reinterpret_cast<const u32x4*>(p + c0);
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (c0 + e < limit) ? (uint32_t)p[c0 + e] : 0u;
    u32x4 v;
    v[0] = h[0] | (h[1] << 16);
    v[1] = h[2] | (h[3] << 16);
    v[2] = h[4] | (h[5] << 16);
    v[3] = h[6] | (h[7] << 16);
    return v;
}

template <int BM, int BN, int IN, int OUT, bool EDGE>
__global__ __launch_bounds__(256, 1) void gemm_mfma_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tilesM, int tilesN, int group_m,
    int vecA, int vecB) {
    constexpr int BK = 64;
    constexpr int AC = BM / 32;        // A chunks per lane per slice
    constexpr int KB = BN / 32;        // B rows (k) per lane per slice: 8 or 4
    constexpr int KG = BK / KB;        // lanes sharing one 8-column B chunk column
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int STAGE = (BM + BN) * 8;   // 16-byte units per LDS stage
    static_assert(KB == 8 || KB == 4, "B transpose block must be 8x8 or 4x8");
    static_assert(BM % 64 == 0 && BN % 128 == 0, "tile");

    __shared__ u32x4 lds[2 * STAGE];

    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    int tm, tn;
    tile_coords(blockIdx.x, tilesM, tilesN, group_m, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int a_row = t >> 3, a_chunk = t & 7;       // A: rows a_row + 32r, chunk a_chunk
    const int b_kg = t % KG, b_nc = t / KG;          // B: rows b_kg*KB + r, columns 8*b_nc..+7

    const uint16_t* Ablk = A + (int64_t)m0 * lda;
    const uint16_t* Bblk = B + n0;

    u32x4 ra[AC], rb[KB];
    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int nk = (K + BK - 1) / BK;

    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int r = 0; r < AC; ++r) {
            const int row = a_row + 32 * r;
            const int kk = k0 + a_chunk * 8;
            if constexpr (!EDGE) {
                ra[r] = *reinterpret_cast<const u32x4*>(Ablk + (int64_t)row * lda + kk);
            } else {
                if (m0 + row < M)
                    ra[r] = load_chunk_masked(Ablk + (int64_t)row * lda, kk, K, vecA);
                else
                    ra[r] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int r = 0; r < KB; ++r) {
            const int kr = k0 + b_kg * KB + r;
            const int nn = b_nc * 8;
            if constexpr (!EDGE) {
                rb[r] = *reinterpret_cast<const u32x4*>(Bblk + (int64_t)kr * ldb + nn);
            } else {
                if (kr < K)
                    rb[r] = load_chunk_masked(Bblk + (int64_t)kr * ldb, nn, N - n0, vecB);
                else
                    rb[r] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };

    auto swrite = [&](int st) {
        u32x4* sA = lds + st * STAGE;
        u32x4* sB = sA + BM * 8;
#pragma unroll
        for (int r = 0; r < AC; ++r) {
            const int row = a_row + 32 * r;
            sA[row * 8 + (a_chunk ^ (row & 7))] = ra[r];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = b_nc * 8 + j;            // n & 7 == j
            if constexpr (KB == 8) {
                u32x4 v;
#pragma unroll
                for (int d = 0; d < 4; ++d) v[d] = pack_col(rb[2 * d], rb[2 * d + 1], j);
                sB[n * 8 + (b_kg ^ j)] = v;
            } else {
                u32x2 v;
#pragma unroll
                for (int d = 0; d < 2; ++d) v[d] = pack_col(rb[2 * d], rb[2 * d + 1], j);
                const int chunk = b_kg >> 1, half = b_kg & 1;
                reinterpret_cast<u32x2*>(sB)[(n * 8 + (chunk ^ j)) * 2 + half] = v;
            }
        }
    };

    if (nk > 0) {
        gload(0);
        swrite(0);
        if (nk > 1) gload(1);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const u32x4* sA = lds + (kt & 1) * STAGE;
        const u32x4* sB = sA + BM * 8;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int ch = 2 * s + (lane >> 5);
            u32x4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WTM + 32 * i + (lane & 31);
                fa[i] = sA[row * 8 + (ch ^ (row & 7))];
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WTN + 32 * j + (lane & 31);
                fb[j] = sB[row * 8 + (ch ^ (row & 7))];
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x16<IN>(fa[i], fb[j], acc[i][j]);
        }
        if (kt + 1 < nk) {
            swrite((kt + 1) & 1);
            if (kt + 2 < nk) gload(kt + 2);
        }
        __syncthreads();
    }

    // Epilogue: fp32 -> output type, one rounding, masked at the edges.
    const int g = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * WTN + 32 * j + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * WTM + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
                if (!EDGE || (row < M && col < N)) store_out<OUT>(C, (int64_t)row * ldc + col, acc[i][j][e]);
            }
        }
    }
}

// C = 0 over the M x N region (K == 0).
template <int OUT>
__global__ __launch_bounds__(256) void zero_fill_kernel(void* C, int64_t ldc, int M, int N) {
    const int64_t total = (int64_t)M * N;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx / N, j = idx - i * N;
        store_out<OUT>(C, i * ldc + j, 0.0f);
    }
}

// ---------------------------------------------------------------- instances
const InstanceInfo kInstances[] = {
    {"mfma_256x256x64", 256, 256, 64, false, 8},
    {"mfma_128x128x64", 128, 128, 64, false, 8},
    {"mfma_256x256x64_edge", 256, 256, 64, true, 8},
    {"mfma_128x128x64_edge", 128, 128, 64, true, 8},
};
const int kNumInstances = sizeof(kInstances) / sizeof(kInstances[0]);

bool instance_supports(int id, const Problem& p) {
    if (id < 0 || id >= kNumInstances) return false;
    const InstanceInfo& in = kInstances[id];
    if (in.edge) return true;
    return p.M % in.bm == 0 && p.N % in.bn == 0 && p.K % in.bk == 0 && p.vecA && p.vecB;
}

template <int BM, int BN, bool EDGE>
static hipError_t launch_tile(const Problem& p, int group_m, hipStream_t s) {
    const int tilesM = (p.M + BM - 1) / BM, tilesN = (p.N + BN - 1) / BN;
    const dim3 grid((unsigned)(tilesM * tilesN)), block(256);
#define DHPT_LAUNCH(IN, OUT)                                                                     \
    hipLaunchKernelGGL((gemm_mfma_kernel<BM, BN, IN, OUT, EDGE>), grid, block, 0, s, p.A, p.lda, \
                       p.B, p.ldb, p.C, p.ldc, p.M, p.N, p.K, tilesM, tilesN, group_m,           \
                       (int)p.vecA, (int)p.vecB)
    switch (p.dtype) {
    case 0: DHPT_LAUNCH(IN_F16, OUT_F32); break;
    case 1: DHPT_LAUNCH(IN_F16, OUT_F16); break;
    case 2: DHPT_LAUNCH(IN_BF16, OUT_F32); break;
    default: DHPT_LAUNCH(IN_BF16, OUT_BF16); break;
    }
#undef DHPT_LAUNCH
    return hipGetLastError();
}

hipError_t launch_instance(int id, const Problem& p, hipStream_t s) {
    const int gm = kInstances[id].group_m;
    switch (id) {
    case 0: return launch_tile<256, 256, false>(p, gm, s);
    case 1: return launch_tile<128, 128, false>(p, gm, s);
    case 2: return launch_tile<256, 256, true>(p, gm, s);
    default: return launch_tile<128, 128, true>(p, gm, s);
    }
}

hipError_t launch_zero_fill(const Problem& p, hipStream_t s) {
    const int64_t total = (int64_t)p.M * p.N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    const dim3 grid((unsigned)blocks), block(256);
    switch (p.dtype) {
    case 0: case 2: hipLaunchKernelGGL(zero_fill_kernel<OUT_F32>, grid, block, 0, s, p.C, p.ldc, p.M, p.N); break;
    case 1: hipLaunchKernelGGL(zero_fill_kernel<OUT_F16>, grid, block, 0, s, p.C, p.ldc, p.M, p.N); break;
    default: hipLaunchKernelGGL(zero_fill_kernel<OUT_BF16>, grid, block, 0, s, p.C, p.ldc, p.M, p.N); break;
    }
    return hipGetLastError();
}

}  // namespace dhpt
