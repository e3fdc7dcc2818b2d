// gemm_pp_kernel.h -- the ping-pong (two wave groups) MFMA kernel template
// for gfx950.  Included only by the instantiation unit gemm_pp.hip.
//
// The factory of "The Asynchronous Kernel: Tensor Cores & TMA" (section "The
// factory"): split the waves of a workgroup into two groups that take turns,
// so that one group keeps the matrix units busy while the other moves data,
// and the epilogue of one runs while the other still multiplies.  On gfx950
// the groups cannot differ in register budget (no per-wave register
// reallocation), so both are alike and alternate roles instead:
//
//   * 512 lanes = 8 waves, two per SIMD (waves w and w + 4 share a SIMD):
//     group g = w / 4 owns output rows 128g .. 128g+127 of the 256x256 tile,
//     wave v = w % 4 of a group owns columns 64v .. 64v+63, a 128x64 fp32
//     accumulator (128 registers, 4x2 blocks of v_mfma_f32_32x32x16);
//   * K in 64-deep slices through two LDS stages laid out exactly as in the
//     256x256 direct-to-LDS kernel (gemm_dl_kernel.h: the same swizzles, the
//     same global_load_lds_dwordx4 copies, now 8 per wave per slice);
//   * every slice is four phases for each wave -- load the fragments of
//     k-steps 0,1 (and issue the copies of the next slice), multiply them,
//     load k-steps 2,3, multiply them -- each phase closed by a workgroup
//     barrier (PH = 2; with PH = 4 a phase covers the whole slice: two
//     phases and two barriers per slice, 96 fragment registers instead of 48).  Group 1 passes one extra barrier at the start, so it runs one
//     phase behind group 0: on every SIMD one wave issues MFMAs while the
//     other issues LDS reads and copies;
//   * copies of slice t+1 go to the other stage from the first phase of
//     slice t (that stage's last readers finished a barrier earlier); group 0
//     waits for its copies before the barrier that closes its fourth phase,
//     group 1 before the one closing its third, which is the same barrier, so
//     slice t+1 is complete before anyone reads it;
//   * the barriers after the last loads are dropped (group 0: its last
//     barrier closes its third phase of the last slice; group 1: its second,
//     the same barrier), so group 0's last multiplies and epilogue overlap
//     group 1's last loads and multiplies.
//
// Whole tiles only (M % 256 == N % 256 == K % 64 == 0), 16-bit inputs, both B
// layouts, plain or general epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.h"

namespace dhpt {
namespace pp {

using namespace dl;

template <int N>
__device__ __forceinline__ void wait_lgkm() {
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

template <int IN, int OUT, bool BT, bool EPI, int PH>
__global__ __launch_bounds__(512, 1) void gemm_pp_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tilesM, int tilesN, int group_m,
    EpiArgs ep) {
#ifdef DHPT_TIMELINE
    const TlStamp tl0 = tl_now();
#endif
    constexpr int BM = 256, BN = 256, BK = 64;
    constexpr int TM = 4, TN = 2;                          // 32x32 blocks per wave: 128 x 64
    constexpr int BROW = 2 * BN;                           // row-major B: bytes per k row
    constexpr int A_BYTES = BM * 128, B_BYTES = BT ? BN * 128 : BK * BROW;
    constexpr int STAGE = A_BYTES + B_BYTES;               // 64 KiB
    constexpr int CA = 4, CB = 4;                          // copies per wave per slice (1 KiB each)
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
    const uint32_t smem_base = (uint32_t)(size_t)(lds_char*)smem;

    const int t = threadIdx.x;
    const int l = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int g = w >> 2, v = w & 3;

    int tm, tn;
    tile_coords(blockIdx.x, tilesM, tilesN, group_m, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    // Copies: wave w fills A stage rows 32w .. 32w+31 (copy i: rows 32w + 8i +
    // l/8, physical chunk l % 8) and, for row-major B, k rows 8w .. 8w+7 (copy
    // i: rows 8w + 2i + l/32, physical chunk l % 32); column-major B like A.
    const char* a_base = reinterpret_cast<const char*>(A) + (int64_t)m0 * lda * 2;
    const char* b_base = reinterpret_cast<const char*>(B) + (BT ? (int64_t)n0 * ldb * 2 : (int64_t)n0 * 2);
    uint32_t a_vo[CA], b_vo[CB];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
        const int r = 32 * w + 8 * i + (l >> 3);
        a_vo[i] = (uint32_t)(((int64_t)r * lda + 8 * ((l & 7) ^ swz_a(r))) * 2);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
        if constexpr (BT) {
            const int r = 32 * w + 8 * i + (l >> 3);
            b_vo[i] = (uint32_t)(((int64_t)r * ldb + 8 * ((l & 7) ^ swz_a(r))) * 2);
        } else {
            const int kr = 8 * w + 2 * i + (l >> 5);
            const int col = 8 * ((l & 31) ^ swz_b(kr));
            b_vo[i] = (uint32_t)(((int64_t)kr * ldb + col) * 2);
        }
    }
    const int64_t a_step = BK * 2, b_step = BT ? (int64_t)BK * 2 : (int64_t)BK * ldb * 2;
    const uint32_t dma_a = smem_base + (32 * w) * 128;
    const uint32_t dma_b = smem_base + A_BYTES + (BT ? (32 * w) * 128 : (8 * w) * BROW);

    // Fragment reads within a stage: A rows 128g + 32i + l%32 (k chunk 2s +
    // l/32, swizzled); B columns 64v + 32j + ... as in the direct-to-LDS kernel.
    const int a_off0 = (128 * g + (l & 31)) * 128;
    const int a_sw = swz_a(l & 31);
    const int gq = l >> 4, ip = l & 15;
    const int b_sw = swz_b(ip >> 2);
    int b_off[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        if constexpr (BT) {
            b_off[j] = A_BYTES + (64 * v + 32 * j + (l & 31)) * 128;
        } else {
            const int n = 64 * v + 32 * j + 16 * (gq & 1) + 4 * (ip & 3);
            b_off[j] = A_BYTES + (8 * (gq >> 1) + (ip >> 2)) * BROW + (((n >> 3) ^ b_sw) * 16) + (n & 7) * 2;
        }
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    static_assert(PH == 2 || PH == 4, "k-steps per phase");
    u32x4 fa[PH][TM];
    u32x4 fbt[PH][TN];
    s16x4 fbh[PH][TN][2];

    // The fragments of k-steps PH*h .. PH*h+PH-1 of the slice in `stage`.
    auto load_half = [&](int stage, int h) {
        const char* st = smem + stage * STAGE;
#pragma unroll
        for (int ks = 0; ks < PH; ++ks) {
            const int s = PH * h + ks;
            const int chunk = (2 * s + (l >> 5)) ^ a_sw;
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[ks][i] = *reinterpret_cast<const u32x4*>(st + a_off0 + i * 32 * 128 + chunk * 16);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (BT) {
                    fbt[ks][j] = *reinterpret_cast<const u32x4*>(st + b_off[j] + chunk * 16);
                } else {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int off = b_off[j] + 16 * s * BROW + hh * 4 * BROW;
                        fbh[ks][j][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4*)((const lds_char*)st + off));
                    }
                }
            }
        }
    };
    auto compute_half = [&]() {
#pragma unroll
        for (int ks = 0; ks < PH; ++ks)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    if constexpr (BT) {
                        acc[i][j] = mfma<IN>(fa[ks][i], fbt[ks][j], acc[i][j]);
                    } else {
                        const u32x2 lo = __builtin_bit_cast(u32x2, fbh[ks][j][0]);
                        const u32x2 hi = __builtin_bit_cast(u32x2, fbh[ks][j][1]);
                        acc[i][j] = mfma<IN>(fa[ks][i], u32x4{lo[0], lo[1], hi[0], hi[1]}, acc[i][j]);
                    }
                }
    };
    auto issue_copies = [&](int stage) {
#pragma unroll
        for (int i = 0; i < CA; ++i) lds_dma16(a_base, a_vo[i], dma_a + stage * STAGE + 1024 * i);
#pragma unroll
        for (int i = 0; i < CB; ++i) lds_dma16(b_base, b_vo[i], dma_b + stage * STAGE + 1024 * i);
        a_base += a_step;
        b_base += b_step;
    };
    // __syncthreads: an LDS-ordering fence and s_barrier (the copies are
    // inline assembly, so its fence adds no wait for them)
    auto barrier = [&]() {
        DL_FENCE();
        __syncthreads();
        DL_FENCE();
    };

    const int nk = K / BK;
    if (nk > 0) {
        issue_copies(0);                 // slice 0, by every wave
        wait_copies();
        barrier();
        if (g == 1) barrier();           // group 1 runs one phase behind
        for (int kt = 0; kt < nk; ++kt) {
            const int stage = kt & 1;
            const bool last = kt == nk - 1;
            if constexpr (PH == 2) {
                // phase 1: fragments of k-steps 0, 1; the copies of the next slice
                load_half(stage, 0);
                if (!last) issue_copies(stage ^ 1);
                wait_lgkm<0>();
                barrier();
                // phase 2: multiply them
                compute_half();
                barrier();
                // phase 3: fragments of k-steps 2, 3
                load_half(stage, 1);
                wait_lgkm<0>();
                if (g == 1) wait_copies();   // group 1's copies of the next slice have landed
                if (!last || g == 0) barrier();
                // phase 4: multiply them
                compute_half();
                if (g == 0) wait_copies();   // group 0's copies of the next slice have landed
                if (!last) barrier();
            } else {
                // phase 1: the fragments of the whole slice; the copies of the next one
                load_half(stage, 0);
                if (!last) issue_copies(stage ^ 1);
                wait_lgkm<0>();
                if (g == 1) wait_copies();   // group 1's copies of the next slice have landed
                if (!last || g == 0) barrier();
                // phase 2: multiply them
                compute_half();
                if (g == 0) wait_copies();   // group 0's copies of the next slice have landed
                if (!last) barrier();
            }
        }
    }

    // Epilogue: each wave its 128 x 64 block, as in the direct-to-LDS kernel.
    const int gl = l >> 5;
    float bias_v[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        bias_v[j] = 0.0f;
        if constexpr (EPI) {
            if (ep.bias != nullptr) bias_v[j] = ep.bias[n0 + 64 * v + 32 * j + (l & 31)];
        }
    }
    auto store_tile = [&](auto read_old) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = n0 + 64 * v + 32 * j + (l & 31);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = m0 + 128 * g + 32 * i + 8 * (e >> 2) + 4 * gl + (e & 3);
                    const int64_t idx = (int64_t)row * ldc + col;
                    float y = acc[i][j][e];
                    if constexpr (EPI) {
                        constexpr bool ro = decltype(read_old)::value;
                        float old = 0.0f;
                        if constexpr (ro) old = load_out<OUT>(C, idx);
                        y = epi_value(y, ep, ro, old, bias_v[j]);
                    }
                    store_out<OUT>(C, idx, y);
                }
            }
        }
    };
    if (EPI && ep.beta != 0.0f)
        store_tile(std::integral_constant<bool, true>{});
    else
        store_tile(std::integral_constant<bool, false>{});
#ifdef DHPT_TIMELINE
    tl_record(ep.timeline, tl0);
#endif
}

template <int IN, int OUT, bool BT, bool EPI, int PH>
static void launch_typed(const Problem& p, int group_m, hipStream_t s) {
    const int tilesM = p.M / 256, tilesN = p.N / 256;
    EpiArgs ep{p.alpha, p.beta, p.bias, p.relu};
#ifdef DHPT_TIMELINE
    ep.timeline = timeline_for((int64_t)tilesM * tilesN * 8);
#endif
    hipLaunchKernelGGL((gemm_pp_kernel<IN, OUT, BT, EPI, PH>), dim3((unsigned)(tilesM * tilesN)), dim3(512), 0, s,
                       p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.M, p.N, p.K, tilesM, tilesN, group_m, ep);
}

template <bool BT, bool EPI, int PH>
static hipError_t launch_family(const Problem& p, int group_m, hipStream_t s) {
    switch (p.dtype) {
    case 0: launch_typed<IN_F16, OUT_F32, BT, EPI, PH>(p, group_m, s); break;
    case 1: launch_typed<IN_F16, OUT_F16, BT, EPI, PH>(p, group_m, s); break;
    case 2: launch_typed<IN_BF16, OUT_F32, BT, EPI, PH>(p, group_m, s); break;
    case 3: launch_typed<IN_BF16, OUT_BF16, BT, EPI, PH>(p, group_m, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pp
}  // namespace dhpt
