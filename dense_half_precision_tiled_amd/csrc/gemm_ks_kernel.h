// gemm_ks_kernel.h -- the k-split-across-waves MFMA kernel template for
// gfx950.  Included only by the instantiation units gemm_ks_*.hip.
//
// For problems whose output has too few 256x256 tiles to occupy the 256 CUs
// (2048^3 has 64), the direct-to-LDS kernel falls back to 128x128 tiles, and
// there each wave owns only a 64x64 accumulator tile: twice the LDS fragment
// bytes per MFMA of the 128x128 wave tile.  This kernel keeps the 128x128
// workgroup tile (256 workgroups at 2048^3) but gives every one of its four
// waves the whole 128x128 tile as its fp32 accumulator, and splits K among
// them instead: wave w multiplies k-step w (16 deep) of every 64-deep slice.
// The four partial tiles are summed through LDS after the last slice, in the
// fixed order wave 0 + wave 1 + wave 2 + wave 3 (a reduce-scatter: wave v
// receives the three other partials of row block v), and each wave then
// writes its 32 rows through the same fused epilogue as the other kernels.
// Nothing leaves the workgroup, so there is no workspace and no cross-CU
// reduction.
//
// Data movement per slice is the 128x128 direct-to-LDS kernel's: the
// workgroup copies a 128x64 A slice and a 64x128 B slice into one LDS stage
// with global_load_lds_dwordx4 (same swizzles, same copy addressing, same
// ds_read_b128 / ds_read_b64_tr_b16 fragment reads); only the fragments each
// wave reads differ.  Stages: a ring of four (4 x 32 KiB).  Slice t's stage is
// free while slice t is multiplied (its fragments were read during slice t-1),
// so the copies of slice t+4 go there and have three slices to land; the
// fragments of slice t+1 are read during slice t.  One workgroup barrier per
// slice publishes slice t+1 and releases stage t.  This is the multi-stage
// copy pipeline of the Ada tensor-core GEMM write-up (its pipeline-stage table), with
// the slice split across waves instead of across output sub-tiles.
//
// EDGE modes as in gemm_dl_kernel.h: dl::EDGE_NONE (M % 128 == N % 128 == 0,
// K % 64 == 0) and dl::EDGE_CLAMP (any M, K; any N for column-major B, N % 8 == 0
// for row-major B; the partial last slice filled through VGPRs with zero
// fill).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.h"

namespace dhpt {
namespace ks {

using namespace dl;

// s_waitcnt vmcnt(n) with n a compile-time constant.
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int IN, int OUT, int EDGE, bool BT, bool EPI>
__global__ __launch_bounds__(256, 1) void gemm_ks_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tilesM, int tilesN, int group_m,
    EpiArgs ep) {
#ifdef DHPT_TIMELINE
    const TlStamp tl0 = tl_now();
#endif
    static_assert(EDGE == dl::EDGE_NONE || EDGE == dl::EDGE_CLAMP, "edge mode");
    constexpr int BM = 128, BN = 128, BK = 64;
    constexpr int TM = 4, TN = 4;                          // 32x32 MFMA blocks: the whole tile
    constexpr int S = TM * TN;                             // MFMAs per wave per slice
    constexpr int NBR = BT ? TN : 2 * TN;                  // B fragment reads per slice
    constexpr int R = TM + NBR;                            // LDS reads per wave per slice
    constexpr int A_BYTES = BM * 128, BROW = 2 * BN, B_BYTES = BK * BROW;   // BT: BN * 128, same
    constexpr int STAGE = A_BYTES + B_BYTES;               // 32 KiB
    constexpr int NST = 4;                                 // stages in the ring (3, 4, 5 measure the same)
    constexpr int CA = BM / 32, CB = BN / 32;              // copies per wave per slice (1 KiB each)
    constexpr int COPIES = CA + CB;
    constexpr int B_ROWS_PER_COPY = 1024 / BROW;           // row-major B: 4 rows per copy
    constexpr int B_CHUNKS = BN / 8;                       // row-major B: 16-byte chunks per row
    constexpr int RED_SLOT = 2 * 4 * 64 * 16;              // reduction: 2 blocks x 4 quads x 64 lanes x 16 B
    static_assert(NST * STAGE <= 160 * 1024, "LDS");
    static_assert(NST * STAGE >= 12 * RED_SLOT, "the reduction's 12 slots reuse the stages");
    __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];
    const uint32_t smem_base = (uint32_t)(size_t)(lds_char*)smem;

    const int t = threadIdx.x;
    const int l = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // this wave's k-step in every slice

    int tm, tn;
    tile_coords(blockIdx.x, tilesM, tilesN, group_m, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // Copy sources: the addressing of the 128x128 direct-to-LDS kernel (a
    // uniform base per operand, advanced one slice at a time, and 32-bit
    // per-lane byte offsets fixed for the whole K loop).
    const char* a_base = reinterpret_cast<const char*>(A) + (int64_t)m0 * lda * 2;
    const char* b_base = reinterpret_cast<const char*>(B) + (BT ? (int64_t)n0 * ldb * 2 : (int64_t)n0 * 2);
    uint32_t a_vo[CA];
    uint32_t b_vo[CB];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int r = (BM / 4) * w + 8 * i + (l >> 3);
        int grow = m0 + r;
        if constexpr (EDGE == dl::EDGE_CLAMP) grow = grow < M ? grow : m0 + (grow - m0) % (M - m0);
        a_vo[i] = (uint32_t)(((int64_t)(grow - m0) * lda + 8 * ((l & 7) ^ swz_a(r))) * 2);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
        if constexpr (BT) {
            const int r = (BN / 4) * w + 8 * i + (l >> 3);
            int gcol = n0 + r;
            if constexpr (EDGE == dl::EDGE_CLAMP) gcol = gcol < N ? gcol : n0 + (gcol - n0) % (N - n0);
            b_vo[i] = (uint32_t)(((int64_t)(gcol - n0) * ldb + 8 * ((l & 7) ^ swz_a(r))) * 2);
        } else {
            const int kr = 16 * w + B_ROWS_PER_COPY * i + l / B_CHUNKS;
            int col = n0 + 8 * ((l % B_CHUNKS) ^ swz_b(kr));
            if constexpr (EDGE == dl::EDGE_CLAMP) col = col + 8 <= N ? col : n0 + (col - n0) % ((N - n0) / 8 * 8);
            b_vo[i] = (uint32_t)(((int64_t)kr * ldb + (col - n0)) * 2);
        }
    }
    const int64_t a_step = (int64_t)BK * 2, b_step = BT ? (int64_t)BK * 2 : (int64_t)BK * ldb * 2;   // bytes
    const uint32_t dma_a = smem_base + ((BM / 4) * w) * 128;
    const uint32_t dma_b = smem_base + A_BYTES + (BT ? ((BN / 4) * w) * 128 : (16 * w) * BROW);

    // Fragment read offsets within a stage for k-step w: A rows 32i + l%32,
    // k chunk 2w + l/32; B as in the direct-to-LDS kernel with k-step w.
    const int a_sw = swz_a(l & 31);
    const int a_off = (l & 31) * 128 + (((2 * w + (l >> 5)) ^ a_sw) * 16);
    const int g = l >> 4, ip = l & 15;
    const int b_sw = swz_b(ip >> 2);
    int b_off[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        if constexpr (BT) {
            b_off[j] = A_BYTES + (32 * j + (l & 31)) * 128 + (((2 * w + (l >> 5)) ^ a_sw) * 16);
        } else {
            const int n = 32 * j + 16 * (g & 1) + 4 * (ip & 3);
            b_off[j] = A_BYTES + (16 * w + 8 * (g >> 1) + (ip >> 2)) * BROW + (((n >> 3) ^ b_sw) * 16) +
                       (n & 7) * 2;
        }
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    u32x4 fa[2][TM];
    u32x4 fbt[2][TN];             // column-major B fragments
    s16x4 fbh[2][TN][2];          // row-major B fragments (two transposing reads each)

    // LDS read q (0 .. R-1) of this wave's k-step from `stage` into buffer
    // `buf`, in consumption order: A0, then B (B0 .. B3, each as lo/hi for
    // row-major B), then A1 .. A3.
    auto read_piece = [&](int stage, int buf, int q) {
        const char* st = smem + stage * STAGE;
        if (q == 0 || q > NBR) {
            const int i = (q == 0) ? 0 : q - NBR;
            fa[buf][i] = *reinterpret_cast<const u32x4*>(st + a_off + i * 32 * 128);
        } else if constexpr (BT) {
            fbt[buf][q - 1] = *reinterpret_cast<const u32x4*>(st + b_off[q - 1]);
        } else {
            const int j = (q - 1) >> 1, h = (q - 1) & 1;
            fbh[buf][j][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)((const lds_char*)st + b_off[j] + h * 4 * BROW));
        }
    };
    // Copy i of a slice into `stage`.  real == false re-copies the previous
    // slice (the sources are not advanced): the filler issued where the
    // slice would lie past K, so that every slice of the loop issues the same
    // copies and waits for the same count; it lands in a stage nobody reads
    // again.
    auto issue_copy = [&](int stage, int i, bool real) {
        // a slice's copies are issued in index order: the bases move on after
        // the last copy of their operand
        if (i < CA) {
            lds_dma16(real ? a_base : a_base - a_step, a_vo[i], dma_a + stage * STAGE + 1024 * i);
            if (i == CA - 1 && real) a_base += a_step;
        } else {
            lds_dma16(real ? b_base : b_base - b_step, b_vo[i - CA], dma_b + stage * STAGE + 1024 * (i - CA));
            if (i == COPIES - 1 && real) b_base += b_step;
        }
    };
    auto mfma1 = [&](int buf, int q) {                 // MFMA q: A block q/TN, B block q%TN
        const int i = q / TN, j = q % TN;
        if constexpr (BT) {
            acc[i][j] = mfma<IN>(fa[buf][i], fbt[buf][j], acc[i][j]);
        } else {
            const u32x2 lo = __builtin_bit_cast(u32x2, fbh[buf][j][0]);
            const u32x2 hi = __builtin_bit_cast(u32x2, fbh[buf][j][1]);
            acc[i][j] = mfma<IN>(fa[buf][i], u32x4{lo[0], lo[1], hi[0], hi[1]}, acc[i][j]);
        }
    };

    // One slice: MFMAs of buffer MB, interleaved one per slot with this
    // slot's share of the R reads of the next slice (stage rstage, buffer
    // MB ^ 1) and of the COPIES copies into cstage.  MB is a compile-time
    // constant so that the fragment buffers stay in registers.
    auto body = [&](auto mb_c, int rstage, int cstage, bool real) {
        constexpr int MB = decltype(mb_c)::value;
#pragma unroll
        for (int q = 0; q < S; ++q) {
            mfma1(MB, q);
#pragma unroll
            for (int x = q * R / S; x < (q + 1) * R / S; ++x) read_piece(rstage, MB ^ 1, x);
#pragma unroll
            for (int c = q * COPIES / S; c < (q + 1) * COPIES / S; ++c) issue_copy(cstage, c, real);
            DL_FENCE();
        }
    };

    const int nk = K / BK;                             // full slices
    if (nk > 0) {
        // Prologue: slices 0 .. 3 into stages 0 .. 3 (fillers past K), wait
        // for slice 0, read its fragments.
#pragma unroll
        for (int st = 0; st < NST; ++st) {
#pragma unroll
            for (int c = 0; c < COPIES; ++c) issue_copy(st, c, st < nk);
        }
        wait_vm<(NST - 1) * COPIES>();
        __syncthreads();
#pragma unroll
        for (int x = 0; x < R; ++x) read_piece(0, 0, x);
        DL_FENCE();

        // Slice kt: the copies of slices kt+2 and kt+3 may still be in
        // flight, those of kt+1 must have landed.  The barrier publishes
        // kt+1 and tells every wave that stage kt (read during kt-1) is free
        // for slice kt+4.  Fragment buffer kt & 1 holds slice kt.  In the
        // last slice the reads of "slice nk" fetch fragments nobody uses.
        auto step = [&](int kt, auto mb_c) {
            wait_vm<(NST - 2) * COPIES>();
            __syncthreads();
            DL_FENCE();
            body(mb_c, (kt + 1) % NST, kt % NST, kt + NST < nk);
        };
        using b0 = std::integral_constant<int, 0>;
        using b1 = std::integral_constant<int, 1>;
        // Two regular loops (even / odd slice count) instead of a tail
        // step after the loop: nothing of the pipeline stays live past it.
        if ((nk & 1) == 0) {
            for (int kt = 0; kt < nk; kt += 2) {
                step(kt, b0{});
                step(kt + 1, b1{});
            }
        } else {
            step(0, b0{});
            for (int kt = 1; kt < nk; kt += 2) {
                step(kt, b1{});
                step(kt + 1, b0{});
            }
        }
    }
    if constexpr (EDGE == dl::EDGE_CLAMP) {
        if (K % BK != 0) {
            // The partial last slice, zero-filled through VGPRs into stage 0
            // (every wave is past the last barrier's reads), then this
            // wave's k-step of it.
            wait_vm<0>();
            __syncthreads();
            fill_stage<BM, BN, BT>(smem, A, lda, B, ldb, M, N, K, m0, n0, nk * BK, t);
            __syncthreads();
#pragma unroll
            for (int x = 0; x < R; ++x) read_piece(0, 0, x);
#pragma unroll
            for (int q = 0; q < S; ++q) mfma1(0, q);
        }
    }

    // Sum of the four partial tiles (a reduce-scatter through LDS): wave v
    // ends with the full sums of row block v (rows 32v .. 32v+31), added in
    // the fixed order wave 0 + wave 1 + wave 2 + wave 3, and stores them.
    // Two rounds of two column blocks; in each, wave w writes its partial of
    // the other waves' row blocks into slot (v, w) (2 blocks x 4 quads x 16
    // bytes per lane, lanes contiguous: 8 KiB; the 12 slots with v != w are
    // numbered 3v + (w < v ? w : w - 1)) and keeps its own in registers.
    wait_vm<0>();
    __syncthreads();                                   // every wave is done with the stages
    const int gl = l >> 5;
    float4* red = reinterpret_cast<float4*>(smem);
    auto slot = [&](int v, int src, int jj, int qd) {      // float4 index of slot (v, src), v != src
        const int sl = 3 * v + (src < v ? src : src > v ? src - 1 : 0);   // src == v: any valid slot
        return (((sl * 2 + jj) * 4 + qd) * 64) + l;
    };
    const bool read_old = EPI && ep.beta != 0.0f;
    const int row_base = m0 + 32 * w + 4 * gl;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int v = 0; v < TM; ++v) {
            if (v == w) continue;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const f32x16& a = acc[v][2 * r + jj];
                    red[slot(v, w, jj, qd)] = float4{a[4 * qd], a[4 * qd + 1], a[4 * qd + 2], a[4 * qd + 3]};
                }
        }
        __syncthreads();
        // Block (w, j): the three other partials from LDS and this wave's
        // own from its accumulators, added in source order.
        auto finish = [&](const f32x16& mine, int jj) {
            const int j = 2 * r + jj;
            float x[16];
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                float4 sum = float4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int src = 0; src < 4; ++src) {
                    const float4 p = src == w ? float4{mine[4 * qd], mine[4 * qd + 1], mine[4 * qd + 2],
                                                       mine[4 * qd + 3]}
                                              : red[slot(w, src, jj, qd)];
                    if (src == 0) sum = p;
                    else { sum.x += p.x; sum.y += p.y; sum.z += p.z; sum.w += p.w; }
                }
                x[4 * qd] = sum.x; x[4 * qd + 1] = sum.y; x[4 * qd + 2] = sum.z; x[4 * qd + 3] = sum.w;
            }
            const int col = n0 + 32 * j + (l & 31);
            float bias_v = 0.0f;
            if constexpr (EPI) {
                if (ep.bias != nullptr && (EDGE == dl::EDGE_NONE || col < N)) bias_v = ep.bias[col];
            }
            if constexpr (EDGE == dl::EDGE_CLAMP) {
                // clamped edges: through a buffer descriptor over the tile's
                // first element, elements outside M x N at an out-of-range
                // offset (dropped), so no element branches
                constexpr int OSZ = OUT == OUT_F32 ? 4 : 2;
                const rsrc_t crs = c_rsrc(static_cast<char*>(C) + ((int64_t)m0 * ldc + n0) * OSZ);
                const int cl = col - n0;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int rl = row_base - m0 + 8 * (e >> 2) + (e & 3);
                    const bool ok = m0 + rl < M && col < N;
                    const uint32_t off = ok ? ((uint32_t)rl * (uint32_t)ldc + (uint32_t)cl) * OSZ : kOutOfRange;
                    float y = x[e];
                    if constexpr (EPI) {
                        const float old = read_old ? load_out_buf<OUT>(crs, off) : 0.0f;
                        y = epi_value(y, ep, read_old, old, bias_v);
                    }
                    store_out_buf<OUT>(crs, off, y);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = row_base + 8 * (e >> 2) + (e & 3);
                    const int64_t idx = (int64_t)row * ldc + col;
                    float y = x[e];
                    if constexpr (EPI) {
                        const float old = read_old ? load_out<OUT>(C, idx) : 0.0f;
                        y = epi_value(y, ep, read_old, old, bias_v);
                    }
                    store_out<OUT, EDGE == dl::EDGE_NONE>(C, idx, y);   // non-temporal on whole tiles
                }
            }
        };
        // w is uniform: one branch per wave, compile-time accumulator indices
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            switch (w) {
            case 0: finish(acc[0][2 * r + jj], jj); break;
            case 1: finish(acc[1][2 * r + jj], jj); break;
            case 2: finish(acc[2][2 * r + jj], jj); break;
            default: finish(acc[3][2 * r + jj], jj); break;
            }
        }
        if (r == 0) __syncthreads();                   // the second pass (r = 1) rewrites the slots
    }
#ifdef DHPT_TIMELINE
    tl_record(ep.timeline, tl0);
#endif
}

template <int IN, int OUT, int EDGE, bool BT, bool EPI>
static void launch_typed(const Problem& p, int group_m, hipStream_t s) {
    const int tilesM = (p.M + 127) / 128, tilesN = (p.N + 127) / 128;
    EpiArgs ep{p.alpha, p.beta, p.bias, p.relu};
#ifdef DHPT_TIMELINE
    ep.timeline = timeline_for((int64_t)tilesM * tilesN * 4);
#endif
    hipLaunchKernelGGL((gemm_ks_kernel<IN, OUT, EDGE, BT, EPI>), dim3((unsigned)(tilesM * tilesN)), dim3(256), 0,
                       s, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.M, p.N, p.K, tilesM, tilesN, group_m, ep);
}

template <int EDGE, bool BT, bool EPI>
static hipError_t launch_dtype(const Problem& p, int group_m, hipStream_t s) {
    switch (p.dtype) {
    case 0: launch_typed<IN_F16, OUT_F32, EDGE, BT, EPI>(p, group_m, s); break;
    case 1: launch_typed<IN_F16, OUT_F16, EDGE, BT, EPI>(p, group_m, s); break;
    case 2: launch_typed<IN_BF16, OUT_F32, EDGE, BT, EPI>(p, group_m, s); break;
    default: launch_typed<IN_BF16, OUT_BF16, EDGE, BT, EPI>(p, group_m, s); break;
    }
    return hipGetLastError();
}

template <bool BT, bool EPI>
static hipError_t launch_family(int edge, const Problem& p, int group_m, hipStream_t s) {
    if (edge == dl::EDGE_NONE) return launch_dtype<dl::EDGE_NONE, BT, EPI>(p, group_m, s);
    if (edge == dl::EDGE_CLAMP) return launch_dtype<dl::EDGE_CLAMP, BT, EPI>(p, group_m, s);
    return hipErrorInvalidValue;
}

}  // namespace ks
}  // namespace dhpt
