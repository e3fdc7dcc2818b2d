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

#include <type_traits>

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

// ----------------------------------------------------------------------------
// Direct-to-LDS kernel (aligned shapes: M % 256 == N % 256 == K % 64 == 0,
// 16-byte aligned operands).
//
// Global -> LDS with global_load_lds_dwordx4: each lane hands 16 bytes of
// global memory to LDS address base + 16 * lane, so a wave fills 1 KiB of LDS
// per instruction without touching VGPRs; the copy is asynchronous and
// completes against vmcnt, the gfx950 counterpart of the cp.async stages of
// the Ada write-up.  Two stages: the loads of slice kt+1 are issued right
// after the barrier that opens slice kt and land while slice kt is multiplied.
//
// LDS layouts (16-byte chunk granularity):
//   A stage: 256 rows x 128 B.  Logical chunk c of row r sits at physical
//     chunk c ^ (r & 7) ^ ((r >> 3) & 1).  The fragment reads (one row per
//     lane, same logical chunk) then cover every 16-byte bank group once per 8
//     rows; measured, they run at ~8.6 clocks per 1 KiB instruction per CU
//     (the LDS's 128 bytes per clock), against 24 without the swizzle.
//   B stage: 64 rows (k) x 512 B (256 n), row-major as in global memory.
//     Logical chunk c of row k sits at physical chunk c ^ 2(k & 3).  Measured
//     on gfx950 (LDS-rate probe, 4 waves per CU), the transposing reads then
//     run at their floor of ~8.3 clocks per instruction per CU; unswizzled
//     rows take 9.0 and a 64-byte-block rotation 10.1.
// The swizzle is applied on the global side: the lane that writes physical
// chunk p of row r fetches logical chunk p ^ swizzle(r).
//
// LDS -> VGPR: A fragments with ds_read_b128 (8 consecutive k of one row);
// B fragments with two ds_read_b64_tr_b16 each.  Within a 16-lane group that
// instruction gives lane i the 4 values of column i of the 4 x 16 block whose
// rows are addressed by lanes 4j + i/4, so lane l ends up holding
// B[k0 .. k0+7][n0 + l % 32] -- the MFMA B operand -- straight from the
// row-major tile (the ldmatrix .trans idea of "mma.sync and ldmatrix", in
// its gfx950 form).
// ----------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_b(int k) { return 2 * (k & 3); }

// One global_load_lds_dwordx4: this lane's 16 bytes at `src` go to LDS byte
// address lds_base + 16 * lane.  Issued through inline assembly so that the
// compiler does not track it: it would otherwise make every later LDS read
// wait for the copy (vmcnt(0)), serialising the next slice's copy with the
// current slice's math.  Completion is awaited explicitly (vmcnt) before the
// barrier that publishes the stage.  M0 has no other user in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_dma_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Keep the scheduler from moving anything across this point: the source order
// below is the issue order.
#define DHPT_FENCE() __builtin_amdgcn_sched_barrier(0)

template <int N>
__device__ __forceinline__ void wait_dma_le() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// 256x256 output tile, BK-deep slices (64 or 32), STAGES LDS stages: the
// copies of slice kt + STAGES - 1 are issued while slice kt is multiplied.
// FD = fragment prefetch distance in k-steps (1 or 2): the LDS reads of
// k-step s + FD are issued while the MFMAs of k-step s run.
template <int IN, int OUT, int BK, int STAGES, int FD = 1>
__global__ __launch_bounds__(256, 1) void gemm_lds_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tilesM, int tilesN, int group_m) {
    static_assert(BK == 64 || BK == 32, "slice depth");
    constexpr int BM = 256, BN = 256;
    constexpr int ROWB = BK * 2;                          // bytes per A row in LDS
    constexpr int A_BYTES = BM * ROWB, B_BYTES = BK * BN * 2;
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    constexpr int KSTEPS = BK / 16;
    constexpr int CPW = BK / 8;                           // copies per wave per slice, for A and for B
    constexpr int COPIES = 2 * CPW;
    constexpr int A_ROWS_PER_COPY = 1024 / ROWB;          // 8 (BK 64) or 16 (BK 32)
    constexpr int A_CHUNKS = ROWB / 16;                   // 8 or 4
    constexpr int B_ROWS_PER_WAVE = BK / 4;
    constexpr int D = STAGES - 1;                         // prefetch distance in slices
    constexpr int NB = (FD == 1) ? 2 : KSTEPS;            // fragment buffers
    static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS");
    static_assert(FD == 1 || (FD == 2 && KSTEPS == 4), "fragment distance");
    __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];
    const uint32_t smem_base = (uint32_t)(size_t)(lds_char*)smem;

    const int l = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 1, wn = w & 1;

    int tm, tn;
    tile_coords(blockIdx.x, tilesM, tilesN, group_m, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // A swizzle (physical 16-byte chunk = logical chunk ^ swa(row)):
    // 128-byte rows: (r & 7) ^ ((r >> 3) & 1); 64-byte rows: (r >> 1) & 3.
    auto swa = [](int r) { return BK == 64 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 1) & 3); };

    // Global sources of this lane's copies.  A copy i of wave w fills rows
    // 64w + A_ROWS_PER_COPY*i + l / A_CHUNKS, physical chunk l % A_CHUNKS;
    // B copy i fills rows B_ROWS_PER_WAVE*w + 2i + l/32, physical chunk l%32.
    const uint16_t* a_src[CPW];
    const uint16_t* b_src[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int r = 64 * w + A_ROWS_PER_COPY * i + l / A_CHUNKS;
        const int c = (l % A_CHUNKS) ^ swa(r);
        a_src[i] = A + (int64_t)(m0 + r) * lda + 8 * c;
        const int kr = B_ROWS_PER_WAVE * w + 2 * i + (l >> 5);
        const int cb = (l & 31) ^ swz_b(kr);
        b_src[i] = B + (int64_t)kr * ldb + n0 + 8 * cb;
    }
    const int64_t b_step = (int64_t)BK * ldb;
    const uint32_t dma_a = smem_base + (64 * w) * ROWB;
    const uint32_t dma_b = smem_base + A_BYTES + (B_ROWS_PER_WAVE * w) * 512;

    // Fragment addresses (bytes within a stage).
    const int a_off0 = (wm * 128 + (l & 31)) * ROWB;
    const int a_sw = swa(l & 31);                           // swa of every row this lane reads
    const int g = l >> 4, ip = l & 15;
    const int b_sw = swz_b(ip >> 2);                        // (k & 3) == (i' >> 2) for every read
    int b_off[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = wn * 128 + 32 * j + 16 * (g & 1) + 4 * (ip & 3);
        b_off[j] = A_BYTES + (8 * (g >> 1) + (ip >> 2)) * 512 + (((n >> 3) ^ b_sw) * 16) + (n & 7) * 2;
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    u32x4 fa[NB][4];               // fragment buffers: k-step s uses buffer s % NB
    s16x4 fbh[NB][4][2];           // the two transposing reads behind each B fragment

    // The 12 LDS reads of one k-step, in the order the next k-step's MFMAs
    // consume them: A0, B0 (two halves), B1, B2, B3, A1, A2, A3.
    auto read_piece = [&](int stage, int s, int buf, int q) {
        const char* st = smem + stage * STAGE_BYTES;
        if (q == 0 || q >= 9) {
            const int i = (q == 0) ? 0 : q - 8;
            const int achunk = (2 * s + (l >> 5)) ^ a_sw;
            fa[buf][i] = *reinterpret_cast<const u32x4*>(st + a_off0 + i * 32 * ROWB + achunk * 16);
        } else {
            const int j = (q - 1) >> 1, h = (q - 1) & 1;
            const int off = b_off[j] + 16 * s * 512 + h * 4 * 512;
            fbh[buf][j][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)((const lds_char*)st + off));
        }
    };
    auto issue_copy = [&](int stage, int i) {          // copy i of COPIES for one slice
        if (i < 0 || i >= COPIES) return;              // never taken: every caller passes 0 .. COPIES-1
        if (i < CPW) {
            lds_dma16(a_src[i], dma_a + stage * STAGE_BYTES + 1024 * i);
            a_src[i] += BK;
        } else {
            lds_dma16(b_src[i - CPW], dma_b + stage * STAGE_BYTES + 1024 * (i - CPW));
            b_src[i - CPW] += b_step;
        }
    };
    auto mfma1 = [&](int buf, int q) {                 // MFMA q of a k-step: A frag q/4, B frag q%4
        const int i = q >> 2, j = q & 3;
        const u32x2 l2 = __builtin_bit_cast(u32x2, fbh[buf][j][0]);
        const u32x2 h2 = __builtin_bit_cast(u32x2, fbh[buf][j][1]);
        acc[i][j] = mfma_32x32x16<IN>(fa[buf][i], u32x4{l2[0], l2[1], h2[0], h2[1]}, acc[i][j]);
    };

    // 16 issue slots: MFMA q of the k-step held in `buf` (if any), then at most
    // one LDS read of the next k-step and at most one copy of a later slice.
    // Copies are spread evenly over the slice's MFMA slots (slot_base numbers
    // this group's first slot within the slice): the per-CU copy path takes
    // about 58 bytes per clock, so a burst of copies would back up and stall
    // the single wave on each SIMD, MFMA pipe and all.
    // With two stages (D == 1) the copies must land within one slice, so they
    // go out early (one per slot, or every other slot with FD == 2).
    constexpr int SPACING = (D >= 2) ? (KSTEPS * 16) / COPIES : ((FD == 2) ? 2 : 16 / COPIES);
    // Every slice issues copies 0 .. COPIES-1 exactly once: slot n of the
    // slice (0 .. 16*KSTEPS-1) issues copy n / SPACING when n % SPACING == 0
    // and n / SPACING < COPIES.
    static_assert(SPACING >= 1 && (COPIES - 1) * SPACING < 16 * KSTEPS, "copy schedule must fit the slice");
    auto copy_at = [](int slot) { return (slot % SPACING == 0 && slot / SPACING < COPIES) ? slot / SPACING : -1; };
    auto units = [&](auto do_mfma, int buf, int rstage, int rs, int rbuf, auto do_copy, int cstage,
                     int slot_base) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            if constexpr (decltype(do_mfma)::value) mfma1(buf, q);
            if (q < 12) read_piece(rstage, rs, rbuf, q);
            if constexpr (decltype(do_copy)::value) {
                const int c = copy_at(slot_base + q);
                if (c >= 0) issue_copy(cstage, c);
            }
            DHPT_FENCE();
        }
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;

    // The copies of slice kt landed for every wave (this wave's: vmcnt; the
    // others': the barrier), and slice kt-1 has been read by everyone.
    // `later` = slices after kt whose copies are already in flight.
    auto open_slice = [&](int later) {
        if (later >= 3) wait_dma_le<3 * COPIES>();
        else if (later == 2) wait_dma_le<2 * COPIES>();
        else if (later == 1) wait_dma_le<COPIES>();
        else wait_dma_le<0>();
        __syncthreads();
        DHPT_FENCE();
    };

    // One slice: the previous slice's last FD k-steps (fragments already in
    // registers) interleaved with this slice's first FD k-steps of reads and
    // the copies of slice kt + D; then k-steps 0 .. KSTEPS-FD-1, each
    // interleaved with the reads of k-step s + FD.  Running the previous
    // slice's last k-steps after the barrier hides the latency of this
    // slice's first reads.
    auto slice = [&](int kt, auto has_prev, auto has_next) {
        const int stage = kt % STAGES;
        const int cstage = (kt + D) % STAGES;
        if constexpr (FD == 1) {
            units(has_prev, 1, stage, 0, 0, has_next, cstage, 0);
#pragma unroll
            for (int s = 0; s < KSTEPS - 1; ++s)
                units(yes{}, s & 1, stage, s + 1, (s + 1) & 1, has_next, cstage, 16 * (s + 1));
        } else {
            // 32 slots: MFMAs of the previous slice's k-steps 2 and 3 with the
            // reads of this slice's k-steps 0 and 1.
#pragma unroll
            for (int q = 0; q < 32; ++q) {
                if constexpr (decltype(has_prev)::value) mfma1(2 + (q >> 4), q & 15);
                if ((q & 15) < 12) read_piece(stage, q >> 4, q >> 4, q & 15);
                if constexpr (decltype(has_next)::value) {
                    const int c = copy_at(q);
                    if (c >= 0) issue_copy(cstage, c);
                }
                DHPT_FENCE();
            }
            units(yes{}, 0, stage, 2, 2, has_next, cstage, 32);
            units(yes{}, 1, stage, 3, 3, has_next, cstage, 48);
        }
    };

    const int nk = K / BK;
    for (int t = 0; t < D && t < nk; ++t)
#pragma unroll
        for (int i = 0; i < COPIES; ++i) issue_copy(t, i);
    // slice 0
    open_slice(nk - 1 < D - 1 ? nk - 1 : D - 1);
    if (D < nk) slice(0, no{}, yes{}); else slice(0, no{}, no{});
    // steady state: copies of slice kt + D are issued
    for (int kt = 1; kt < nk - D; ++kt) {
        open_slice(D - 1);
        slice(kt, yes{}, yes{});
    }
    // last D slices (or fewer): no more copies
    for (int kt = (nk - D > 1 ? nk - D : 1); kt < nk; ++kt) {
        open_slice(nk - 1 - kt);
        slice(kt, yes{}, no{});
    }
    if constexpr (FD == 2) {
#pragma unroll
        for (int q = 0; q < 16; ++q) mfma1(2, q);     // last two k-steps of the last slice
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) mfma1(FD == 2 ? 3 : 1, q);

    const int gl = l >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 128 + 32 * j + (l & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * gl + (e & 3);
                store_out<OUT>(C, (int64_t)row * ldc + col, acc[i][j][e]);
            }
        }
    }
}

// ----------------------------------------------------------------------------
// Eight-wave kernel: 512 lanes, two waves per SIMD, 2 x 4 grid of 128 x 64
// wave tiles over the 256 x 256 output tile (128 fp32 accumulators per lane).
// Same LDS stages, swizzles and copies as gemm_lds_kernel.  With a second
// wave on every SIMD, one wave's MFMAs run while the other waits on LDS or
// on the barrier, and twice as many fragment reads are in flight: measured on
// gfx950, LDS throughput grows with the reads in flight (ds_read_b128 about
// 100 / 187 / 263 bytes per clock per CU with 4 / 8 / 16 waves; the
// transposing read 62 / 120 / 155).
// ----------------------------------------------------------------------------
template <int IN, int OUT, int FD>
__global__ __launch_bounds__(512, 1) void gemm_lds8_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tilesM, int tilesN, int group_m) {
    constexpr int BM = 256, BN = 256, BK = 64, ROWB = 128;
    constexpr int A_BYTES = BM * ROWB, B_BYTES = BK * BN * 2;
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    constexpr int KSTEPS = 4;
    constexpr int CPW = 4;                        // copies per wave per slice, for A and for B
    constexpr int COPIES = 2 * CPW;
    constexpr int NB = FD + 1;                    // fragment buffers (k-step s uses buffer s % NB)
    static_assert(FD == 1 || FD == 2, "fragment distance");
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];
    const uint32_t smem_base = (uint32_t)(size_t)(lds_char*)smem;

    const int l = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 2, wn = w & 3;

    int tm, tn;
    tile_coords(blockIdx.x, tilesM, tilesN, group_m, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // Copies: A copy i of wave w fills rows 32w + 8i + l/8 (physical chunk l%8);
    // B copy i fills rows 8w + 2i + l/32 (physical chunk l%32).
    const uint16_t* a_src[CPW];
    const uint16_t* b_src[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int r = 32 * w + 8 * i + (l >> 3);
        a_src[i] = A + (int64_t)(m0 + r) * lda + 8 * ((l & 7) ^ swz_a(r));
        const int kr = 8 * w + 2 * i + (l >> 5);
        b_src[i] = B + (int64_t)kr * ldb + n0 + 8 * ((l & 31) ^ swz_b(kr));
    }
    const int64_t b_step = (int64_t)BK * ldb;
    const uint32_t dma_a = smem_base + (32 * w) * ROWB;
    const uint32_t dma_b = smem_base + A_BYTES + (8 * w) * 512;

    const int a_off0 = (wm * 128 + (l & 31)) * ROWB;
    const int a_sw = swz_a(l & 31);
    const int g = l >> 4, ip = l & 15;
    const int b_sw = swz_b(ip >> 2);
    int b_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int n = wn * 64 + 32 * j + 16 * (g & 1) + 4 * (ip & 3);
        b_off[j] = A_BYTES + (8 * (g >> 1) + (ip >> 2)) * 512 + (((n >> 3) ^ b_sw) * 16) + (n & 7) * 2;
    }

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    u32x4 fa[NB][4];
    s16x4 fbh[NB][2][2];

    // The 8 LDS reads of one k-step in consumption order: A0, B0 lo/hi,
    // B1 lo/hi, A1, A2, A3.
    auto read_piece = [&](int stage, int s, int buf, int q) {
        const char* st = smem + stage * STAGE_BYTES;
        if (q == 0 || q >= 5) {
            const int i = (q == 0) ? 0 : q - 4;
            const int achunk = (2 * s + (l >> 5)) ^ a_sw;
            fa[buf][i] = *reinterpret_cast<const u32x4*>(st + a_off0 + i * 32 * ROWB + achunk * 16);
        } else {
            const int j = (q - 1) >> 1, h = (q - 1) & 1;
            const int off = b_off[j] + 16 * s * 512 + h * 4 * 512;
            fbh[buf][j][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)((const lds_char*)st + off));
        }
    };
    auto issue_copy = [&](int stage, int i) {
        if (i < 0 || i >= COPIES) return;              // never taken: every caller passes 0 .. COPIES-1
        if (i < CPW) {
            lds_dma16(a_src[i], dma_a + stage * STAGE_BYTES + 1024 * i);
            a_src[i] += BK;
        } else {
            lds_dma16(b_src[i - CPW], dma_b + stage * STAGE_BYTES + 1024 * (i - CPW));
            b_src[i - CPW] += b_step;
        }
    };
    auto mfma1 = [&](int buf, int q) {                 // MFMA q of a k-step: A frag q/2, B frag q%2
        const int i = q >> 1, j = q & 1;
        const u32x2 l2 = __builtin_bit_cast(u32x2, fbh[buf][j][0]);
        const u32x2 h2 = __builtin_bit_cast(u32x2, fbh[buf][j][1]);
        acc[i][j] = mfma_32x32x16<IN>(fa[buf][i], u32x4{l2[0], l2[1], h2[0], h2[1]}, acc[i][j]);
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;

    // 8 issue slots per k-step: MFMA q, one read of a later k-step, and (in
    // the first k-step of the slice) one copy of the next slice.
    auto units = [&](auto do_mfma, int buf, int rstage, int rs, int rbuf, auto do_copy, int cstage) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if constexpr (decltype(do_mfma)::value) mfma1(buf, q);
            read_piece(rstage, rs, rbuf, q);
            if constexpr (decltype(do_copy)::value) issue_copy(cstage, q);
            DHPT_FENCE();
        }
    };

    // Slice kt (k-steps 0..3 of stage kt&1): the previous slice's last FD
    // k-steps run right after the barrier, interleaved with this slice's
    // first FD k-steps of reads and the next slice's copies.
    auto slice = [&](int kt, auto has_prev, auto has_next) {
        const int stage = kt & 1;
        wait_dma_all();
        __syncthreads();
        DHPT_FENCE();
        if constexpr (FD == 1) {
            units(has_prev, 3 % NB, stage, 0, 0, has_next, stage ^ 1);
#pragma unroll
            for (int s = 0; s < KSTEPS - 1; ++s) units(yes{}, s % NB, stage, s + 1, (s + 1) % NB, no{}, 0);
        } else {
            // buffers: k-step s of slice kt uses (4kt + s) % 3; with four steps
            // per slice that is (kt + s) % 3.
            const int o = kt % 3;
            units(has_prev, (o + 2) % 3, stage, 0, o, has_next, stage ^ 1);          // prev step 2
            units(has_prev, (o + 0) % 3, stage, 1, (o + 1) % 3, no{}, 0);           // prev step 3
#pragma unroll
            for (int s = 0; s < KSTEPS - 2; ++s)
                units(yes{}, (o + s) % 3, stage, s + 2, (o + s + 2) % 3, no{}, 0);
        }
    };

    const int nk = K / BK;
#pragma unroll
    for (int i = 0; i < COPIES; ++i) issue_copy(0, i);
    if (nk > 1) {
        slice(0, no{}, yes{});
        for (int kt = 1; kt < nk - 1; ++kt) slice(kt, yes{}, yes{});
        slice(nk - 1, yes{}, no{});
    } else {
        slice(0, no{}, no{});
    }
    if constexpr (FD == 1) {
#pragma unroll
        for (int q = 0; q < 8; ++q) mfma1(3 % NB, q);
    } else {
        const int o = (nk - 1) % 3;
#pragma unroll
        for (int q = 0; q < 8; ++q) mfma1((o + 2) % 3, q);
#pragma unroll
        for (int q = 0; q < 8; ++q) mfma1(o, q);
    }

    const int gl = l >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + 32 * j + (l & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * gl + (e & 3);
                store_out<OUT>(C, (int64_t)row * ldc + col, acc[i][j][e]);
            }
        }
    }
}

// ----------------------------------------------------------------------------
// Variant with B transposed on its way into LDS.  A is copied global -> LDS
// as above; B goes global -> VGPR (one 8 x 8 block of 16-bit values per lane,
// eight 16-byte loads of consecutive rows), is transposed with byte
// permutes, and is written k-contiguous ([n][k], the same swizzled 128-byte
// rows as A).  Both MFMA operands are then read with ds_read_b128, whose LDS
// cost per byte is half that of the transposing read.
// ----------------------------------------------------------------------------
template <int IN, int OUT>
__global__ __launch_bounds__(256, 1) void gemm_ldsbt_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tilesM, int tilesN, int group_m) {
    constexpr int BM = 256, BN = 256, BK = 64, ROWB = 128;
    constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];
    const uint32_t smem_base = (uint32_t)(size_t)(lds_char*)smem;

    const int l = threadIdx.x & 63;
    const int t = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 1, wn = w & 1;

    int tm, tn;
    tile_coords(blockIdx.x, tilesM, tilesN, group_m, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // A copies: copy i of wave w fills rows 64w + 8i + l/8, physical chunk l%8.
    const uint16_t* a_src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = 64 * w + 8 * i + (l >> 3);
        a_src[i] = A + (int64_t)(m0 + r) * lda + 8 * ((l & 7) ^ swz_a(r));
    }
    const uint32_t dma_a = smem_base + (64 * w) * ROWB;
    // B block of this lane: rows 8*kb .. 8*kb+7 of the slice, columns 8*nc .. +7.
    const int kb = t & 7, nc = t >> 3;
    const uint16_t* b_src = B + (int64_t)(8 * kb) * ldb + n0 + 8 * nc;
    const int64_t b_step = (int64_t)BK * ldb;
    int b_dst[8];                                   // byte offsets of the 8 transposed chunks
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int n = 8 * nc + j;
        b_dst[j] = A_BYTES + n * ROWB + 16 * (kb ^ swz_a(n));
    }

    const int a_off0 = (wm * 128 + (l & 31)) * ROWB;
    const int b_off0 = A_BYTES + (wn * 128 + (l & 31)) * ROWB;
    const int f_sw = swz_a(l & 31);                 // swizzle of every fragment row this lane reads

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    u32x4 fa[2][4], fb[2][4];
    u32x4 rb[8];

    // The 8 LDS reads of one k-step in consumption order: A0, B0..B3, A1..A3.
    auto read_piece = [&](int stage, int s, int buf, int q) {
        const char* st = smem + stage * STAGE_BYTES;
        const int chunk16 = ((2 * s + (l >> 5)) ^ f_sw) * 16;
        if (q == 0 || q >= 5) {
            const int i = (q == 0) ? 0 : q - 4;
            fa[buf][i] = *reinterpret_cast<const u32x4*>(st + a_off0 + i * 32 * ROWB + chunk16);
        } else {
            const int j = q - 1;
            fb[buf][j] = *reinterpret_cast<const u32x4*>(st + b_off0 + j * 32 * ROWB + chunk16);
        }
    };
    auto issue_a_copy = [&](int stage, int i) {
        lds_dma16(a_src[i], dma_a + stage * STAGE_BYTES + 1024 * i);
        a_src[i] += BK;
    };
    auto load_b_row = [&](int r) {
        rb[r] = *reinterpret_cast<const u32x4*>(b_src + (int64_t)r * ldb);
        if (r == 7) b_src += b_step;
    };
    auto write_b_col = [&](int stage, int j) {       // column j of the 8x8 block, k contiguous
        u32x4 v;
#pragma unroll
        for (int d = 0; d < 4; ++d) v[d] = pack_col(rb[2 * d], rb[2 * d + 1], j);
        *reinterpret_cast<u32x4*>(smem + stage * STAGE_BYTES + b_dst[j]) = v;
    };
    auto mfma1 = [&](int buf, int q) {
        const int i = q >> 2, j = q & 3;
        acc[i][j] = mfma_32x32x16<IN>(fa[buf][i], fb[buf][j], acc[i][j]);
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;

    // Slots of one k-step: MFMA q, then (slots 0..7) one read of the next
    // k-step; the prefetch of the next slice rides in the first k-step (A
    // copy and B row load per slot), its transposed B writes in the last.
    auto units = [&](auto do_mfma, int buf, int rstage, int rs, int rbuf, auto do_fetch, auto do_bwrite,
                     int nstage) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            if constexpr (decltype(do_mfma)::value) mfma1(buf, q);
            if (q < 8) read_piece(rstage, rs, rbuf, q);
            if constexpr (decltype(do_fetch)::value) {
                if (q < 8) issue_a_copy(nstage, q);
                else load_b_row(q - 8);
            }
            if constexpr (decltype(do_bwrite)::value) {
                if (q >= 8) write_b_col(nstage, q - 8);
            }
            DHPT_FENCE();
        }
    };

    // Slice kt: barrier (A copies and B writes of slice kt visible, slice
    // kt-1 fully read); the previous slice's last k-step with this slice's
    // first reads and the fetch of slice kt+1; k-steps 0..2 with the reads of
    // the following k-step; slice kt+1's B block is written during k-step 2.
    auto slice = [&](int kt, auto has_prev, auto has_next) {
        const int stage = kt & 1, nstage = stage ^ 1;
        wait_dma_all();
        __syncthreads();
        DHPT_FENCE();
        units(has_prev, 1, stage, 0, 0, has_next, no{}, nstage);
        units(yes{}, 0, stage, 1, 1, no{}, no{}, nstage);
        units(yes{}, 1, stage, 2, 0, no{}, no{}, nstage);
        units(yes{}, 0, stage, 3, 1, no{}, has_next, nstage);
    };

    const int nk = K / BK;
    // prologue: slice 0 in stage 0
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_a_copy(0, i);
#pragma unroll
    for (int r = 0; r < 8; ++r) load_b_row(r);
#pragma unroll
    for (int j = 0; j < 8; ++j) write_b_col(0, j);
    if (nk > 1) {
        slice(0, no{}, yes{});
        for (int kt = 1; kt < nk - 1; ++kt) slice(kt, yes{}, yes{});
        slice(nk - 1, yes{}, no{});
    } else {
        slice(0, no{}, no{});
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) mfma1(1, q);

    const int gl = l >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 128 + 32 * j + (l & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * gl + (e & 3);
                store_out<OUT>(C, (int64_t)row * ldc + col, acc[i][j][e]);
            }
        }
    }
}

// ---------------------------------------------------------------- instances
const InstanceInfo kInstances[] = {
    {"mfma_256x256x64_lds2", 256, 256, 64, false, 8, REQ_TILE_VEC},
    {"mfma_128x128x64", 128, 128, 64, false, 8, REQ_TILE_VEC},
    {"mfma_256x256x64_edge", 256, 256, 64, true, 8, REQ_ANY},
    {"mfma_128x128x64_edge", 128, 128, 64, true, 8, REQ_ANY},
    {"mfma_256x256x64", 256, 256, 64, false, 8, REQ_TILE_VEC},
    {"mfma_256x256x32_lds4", 256, 256, 32, false, 8, REQ_TILE_VEC},
    {"mfma_256x256x32_lds5", 256, 256, 32, false, 8, REQ_TILE_VEC},
    {"mfma_256x256x64_ldsbt", 256, 256, 64, false, 8, REQ_TILE_VEC},
    {"mfma_256x256x64_lds2_fd2", 256, 256, 64, false, 8, REQ_TILE_VEC},
    {"mfma_256x256x64_w8", 256, 256, 64, false, 8, REQ_TILE_VEC},
    {"dl_256x256x64_fd2", 256, 256, 64, false, 8, REQ_TILE},
    {"dl_256x256x64_fd2_edge", 256, 256, 64, true, 8, REQ_N8},
    {"dl_128x128x64_fd1", 128, 128, 64, false, 8, REQ_TILE},
    {"dl_128x128x64_fd1_edge", 128, 128, 64, true, 8, REQ_N8},
    {"dl_128x128x64_fd2", 128, 128, 64, false, 8, REQ_TILE},
    {"dl_128x128x64_fd2_edge", 128, 128, 64, true, 8, REQ_N8},
    {"dl_256x256x64_fd1", 256, 256, 64, false, 8, REQ_TILE},
    {"dl_256x256x64_fd1_edge", 256, 256, 64, true, 8, REQ_N8},
};
const int kNumInstances = sizeof(kInstances) / sizeof(kInstances[0]);

bool instance_supports(int id, const Problem& p) {
    if (id < 0 || id >= kNumInstances) return false;
    const InstanceInfo& in = kInstances[id];
    const bool tiled = p.M % in.bm == 0 && p.N % in.bn == 0 && p.K % in.bk == 0;
    switch (in.req) {
    case REQ_ANY: return true;
    case REQ_TILE_VEC: return tiled && p.vecA && p.vecB;
    case REQ_TILE: return tiled;
    case REQ_N8: return p.N % 8 == 0 && p.N >= 8;
    default: return false;
    }
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

template <int IN, int OUT, int BK, int STAGES, int FD>
static void launch_lds_typed(const Problem& p, int group_m, hipStream_t s) {
    const int tilesM = p.M / 256, tilesN = p.N / 256;
    hipLaunchKernelGGL((gemm_lds_kernel<IN, OUT, BK, STAGES, FD>), dim3((unsigned)(tilesM * tilesN)),
                       dim3(256), 0, s, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.M, p.N, p.K, tilesM, tilesN,
                       group_m);
}

template <int IN, int OUT>
static void launch_ldsbt_typed(const Problem& p, int group_m, hipStream_t s) {
    const int tilesM = p.M / 256, tilesN = p.N / 256;
    hipLaunchKernelGGL((gemm_ldsbt_kernel<IN, OUT>), dim3((unsigned)(tilesM * tilesN)), dim3(256), 0, s,
                       p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.M, p.N, p.K, tilesM, tilesN, group_m);
}

template <int IN, int OUT, int FD>
static void launch_lds8_typed(const Problem& p, int group_m, hipStream_t s) {
    const int tilesM = p.M / 256, tilesN = p.N / 256;
    hipLaunchKernelGGL((gemm_lds8_kernel<IN, OUT, FD>), dim3((unsigned)(tilesM * tilesN)), dim3(512), 0, s,
                       p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.M, p.N, p.K, tilesM, tilesN, group_m);
}

template <int FD>
static hipError_t launch_lds8(const Problem& p, int group_m, hipStream_t s) {
    switch (p.dtype) {
    case 0: launch_lds8_typed<IN_F16, OUT_F32, FD>(p, group_m, s); break;
    case 1: launch_lds8_typed<IN_F16, OUT_F16, FD>(p, group_m, s); break;
    case 2: launch_lds8_typed<IN_BF16, OUT_F32, FD>(p, group_m, s); break;
    default: launch_lds8_typed<IN_BF16, OUT_BF16, FD>(p, group_m, s); break;
    }
    return hipGetLastError();
}

static hipError_t launch_ldsbt(const Problem& p, int group_m, hipStream_t s) {
    switch (p.dtype) {
    case 0: launch_ldsbt_typed<IN_F16, OUT_F32>(p, group_m, s); break;
    case 1: launch_ldsbt_typed<IN_F16, OUT_F16>(p, group_m, s); break;
    case 2: launch_ldsbt_typed<IN_BF16, OUT_F32>(p, group_m, s); break;
    default: launch_ldsbt_typed<IN_BF16, OUT_BF16>(p, group_m, s); break;
    }
    return hipGetLastError();
}

template <int BK, int STAGES, int FD = 1>
static hipError_t launch_lds(const Problem& p, int group_m, hipStream_t s) {
    switch (p.dtype) {
    case 0: launch_lds_typed<IN_F16, OUT_F32, BK, STAGES, FD>(p, group_m, s); break;
    case 1: launch_lds_typed<IN_F16, OUT_F16, BK, STAGES, FD>(p, group_m, s); break;
    case 2: launch_lds_typed<IN_BF16, OUT_F32, BK, STAGES, FD>(p, group_m, s); break;
    default: launch_lds_typed<IN_BF16, OUT_BF16, BK, STAGES, FD>(p, group_m, s); break;
    }
    return hipGetLastError();
}

hipError_t launch_instance(int id, const Problem& p, hipStream_t s) {
    const int gm = kInstances[id].group_m;
    switch (id) {
    case 0: return launch_lds<64, 2>(p, gm, s);
    case 5: return launch_lds<32, 4>(p, gm, s);
    case 6: return launch_lds<32, 5>(p, gm, s);
    case 7: return launch_ldsbt(p, gm, s);
    case 8: return launch_lds<64, 2, 2>(p, gm, s);
    case 9: return launch_lds8<1>(p, gm, s);
    case 10: return launch_dl(256, 2, false, p, gm, s);
    case 11: return launch_dl(256, 2, true, p, gm, s);
    case 12: return launch_dl(128, 1, false, p, gm, s);
    case 13: return launch_dl(128, 1, true, p, gm, s);
    case 14: return launch_dl(128, 2, false, p, gm, s);
    case 15: return launch_dl(128, 2, true, p, gm, s);
    case 16: return launch_dl(256, 1, false, p, gm, s);
    case 17: return launch_dl(256, 1, true, p, gm, s);
    case 4: return launch_tile<256, 256, false>(p, gm, s);
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
