// gemm_dl_kernel.h -- the direct-to-LDS MFMA kernel template for gfx950.
// Included only by the instantiation units gemm_dl_*.hip.
//
// Per workgroup: 4 waves in a 2x2 grid, each owning a (BM/2) x (BN/2) fp32
// accumulator tile built from v_mfma_f32_32x32x16_{f16,bf16} (16-bit inputs;
// the 8-bit form below).  K is streamed in 64-deep slices through two LDS
// stages:
//   * global -> LDS with global_load_lds_dwordx4 (16 bytes per lane, 1 KiB
//     per wave instruction, no VGPR staging; a uniform scalar base per
//     operand plus a fixed 32-bit per-lane offset below 2^31, so larger
//     problems go to EDGE_MASKED), issued while the previous
//     slice is multiplied -- the multi-stage copy pipeline of the Ada
//     tensor-core GEMM write-up (its pipeline-stage table) and the acquire / copy /
//     wait / release loop of "GEMM From Naive CUDA to Tensor Cores" ("Where
//     asynchronous copies and TMA take over"), with vmcnt as the wait and one
//     workgroup barrier per slice as both the publish and the release;
//   * A stage: BM rows x 128 bytes (64 k); logical 16-byte chunk c of row r
//     at physical chunk c ^ (r & 7) ^ ((r >> 3) & 1).  The XOR-of-chunks idea
//     of "The Asynchronous Kernel: Tensor Cores & TMA" ("The XOR that unties
//     the banks"), with the row function picked by measuring LDS read rates;
//   * B stage, row-major B (K x N in memory): 64 rows x 2*BN bytes, row-major
//     like global memory; chunk c of row k at c ^ 2(k & 3).  B fragments come
//     from two ds_read_b64_tr_b16 each, which give lane l the 8 values of k
//     for column l % 32 straight from the row-major tile (the transposing
//     load of "mma.sync and ldmatrix", gfx950 form);
//   * B stage, column-major B (BT, N x K in memory, the "TN" layout of the Ada
//     write-up's operand-layout choice, A row-major and B column-major): BN rows x 128
//     bytes, copied and swizzled exactly like A; B fragments are then plain
//     ds_read_b128 like A's;
//   * A fragments: ds_read_b128 (8 consecutive k of one row);
//   * issue order fixed in source (sched_barrier): one MFMA per slot followed
//     by the slot's share of next-k-step reads and next-slice copies; the last
//     FD k-steps of a slice run after the next barrier;
//   * epilogue: fp32 -> output type with one rounding, stores masked at the
//     M and N edges ("Turn global loads into shared tiles": predicate the
//     store, not the barriers).  With EPI, the value stored is
//     act(alpha * acc + beta * C_old + bias[col]) computed in fp32 before the
//     one rounding (the fused bias + ReLU epilogue of the Ada write-up and
//     the general C <- alpha*A*B + beta*C of the naive-to-tensor-core page);
//     C_old is read only when beta != 0.
//
// 8-bit float inputs (IN_E4M3, IN_E5M2): a slice is still 128 bytes of every
// A row (and column-major B row), now 128 values of k, multiplied as two
// 64-deep k-steps of v_mfma_f32_32x32x64_f8f6f4.  A lane's fragment is 32
// consecutive k, the same k for A and B: two ds_read_b128 of a swizzled A (or
// column-major B) row, or, for row-major B (128 rows x BN bytes, chunk c of
// row k at c ^ swz_b8(k)), four ds_read_b64_tr_b8, each handing every lane 8
// values of k of its column.  The fragments of the next k-step are read while
// the current one is multiplied (FD == 1: at 64 deep a k-step is as long as
// two of the 16-bit ones).  Copies and epilogue are those of the 16-bit
// kernel.  The 8-bit float of the Ada write-up's precision notes, built here
// for gfx950's double-rate 8-bit MFMA.
//
// EDGE modes (BK = 64 for 16-bit inputs, 128 for 8-bit ones):
//   EDGE_NONE:  M % BM == N % BN == K % BK == 0.
//   EDGE_CLAMP: any M, K; any N for column-major B, N % 8 == 0 (N % 16 == 0
//     for 8-bit inputs) for row-major B.  Rows of A (and of column-major B)
//     past the edge and 16-byte column chunks of row-major B past N are read
//     from valid ones of the same tile, wrapped around (m0 + (r - m0) mod
//     (M - m0)): those values only reach outputs that are never stored, and
//     wrapping keeps the lanes of a copy on distinct addresses (clamping
//     them all to the last row made the edge tiles of a one-wave launch its
//     slowest).  A partial last slice (K % BK != 0) is filled through
//     VGPRs with element-exact zero fill.
//   EDGE_MASKED: any shape.  Every slice is filled through VGPRs with
//     element-exact zero fill (no asynchronous copies, one stage, 64-bit
//     addresses); the fallback for row-major B with N % 8 != 0 (N % 16 != 0
//     for 8-bit inputs) and for leading dimensions whose copy offsets would
//     reach 2^31 bytes.
// 16-byte loads from any byte address return the exact bytes on gfx950
// (pinned by a probe test), so misaligned rows and leading dimensions stay on
// the vector paths.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.h"

namespace dhpt {
namespace dl {

// LDS bytes of one workgroup: NSTAGE stages of an A slice (BM rows x 128
// bytes) and a B slice (column-major: BN rows x 128 bytes; row-major: 128 /
// element-size rows of BN elements), one stage for EDGE_MASKED.
template <int IN, int BM, int BN, int EDGE, bool BT>
constexpr int dl_lds_bytes() {
    constexpr int ESZ = kIn8<IN> ? 1 : 2;
    return (EDGE == EDGE_MASKED ? 1 : 2) * (BM * 128 + (BT ? BN * 128 : (128 / ESZ) * ESZ * BN));
}

// One output tile, rows m0 .. m0+BM-1 and columns n0 .. n0+BN-1, by the 256
// lanes of the calling workgroup, with `smem` (dl_lds_bytes bytes, 1 KiB
// aligned) as its LDS stages.  `tid` is threadIdx.x (the persistent kernel
// passes a value the compiler cannot move out of its tile loop, so that the
// lane offsets derived from it are recomputed per tile instead of being
// kept live across the accumulator-heavy main loop).  On return every wave
// has issued its stores and no wave reads `smem` any more once all have
// returned.  NTC: store the tile with non-temporal stores.  The whole-tile
// kernels do (the host gives them only C whose rows start on 64-byte
// boundaries, so that every store instruction writes whole 64-byte
// segments); the edge kernels, whose C rows may sit at any 2-byte offset,
// and the split-K kernel's fp32 partial tiles, which its second kernel reads
// back, keep the default cache policy.  ROWS: unmasked tiles store whole
// 64-column row pieces (the lane exchange in the epilogue below); the
// persistent kernel, whose tile loop keeps more registers live, does not
// (with it its epilogue spilled to scratch).
template <int IN, int OUT, int BM, int BN, int FD, int EDGE, bool BT, bool EPI, bool NTC = false, bool ROWS = false>
__device__ __forceinline__ void dl_tile(
    char* smem, const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int m0, int n0, const EpiArgs& ep, int tid) {
    static_assert((BM == 256 && BN == 256) || (BM == 128 && BN == 128) || (BM == 64 && BN == 64), "tile");
    static_assert(FD == 1 || FD == 2, "fragment prefetch distance");
    constexpr bool F8 = kIn8<IN>;
    static_assert(!F8 || FD == 1, "8-bit inputs: fragment prefetch one k-step");
    constexpr int ESZ = F8 ? 1 : 2;                       // bytes per input element
    constexpr int BK = F8 ? 128 : 64, KSTEPS = F8 ? 2 : 4;   // k per slice (128 bytes of a row), MFMA k-steps
    constexpr int RPF = F8 ? 2 : 1;                       // ds_read_b128 per A (or column-major B) fragment
    constexpr int WM = BM / 2, WN = BN / 2;               // wave tile
    constexpr int TM = WM / 32, TN = WN / 32;             // MFMA blocks per wave
    constexpr int S = TM * TN;                            // MFMAs (issue slots) per k-step
    constexpr int PB = BT ? RPF : (F8 ? 4 : 2);           // LDS reads per B fragment
    constexpr int NBR = PB * TN;                          // B reads per k-step
    constexpr int R = RPF * TM + NBR;                     // LDS reads per k-step
    constexpr int BROW = ESZ * BN;                        // row-major B: bytes per k row
    constexpr int A_BYTES = BM * 128, B_BYTES = BT ? BN * 128 : (128 / ESZ) * BROW;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int NSTAGE = EDGE == EDGE_MASKED ? 1 : 2;
    constexpr int CA = BM / 32, CB = BN / 32;             // copies per wave per slice (1 KiB each)
    constexpr int COPIES = CA + CB;
    constexpr int B_ROWS_PER_COPY = 1024 / BROW;          // row-major B: k rows per 1 KiB copy
    constexpr int B_CHUNKS = BROW / 16;                   // row-major B: 16-byte chunks per row
    constexpr int B_ROWS_PER_WAVE = (128 / ESZ) / 4;      // row-major B: k rows each wave copies
    constexpr int NB = (FD == 1) ? 2 : 4;                 // fragment buffers
    static_assert(NSTAGE * STAGE == dl_lds_bytes<IN, BM, BN, EDGE, BT>(), "LDS size");
    const uint32_t smem_base = (uint32_t)(size_t)(lds_char*)smem;

    const int t = tid;
    const int l = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = w >> 1, wn = w & 1;

    // Copy sources.  A copy i of wave w fills stage rows (BM/4)w + 8i + l/8,
    // physical chunk l%8; column-major B the same over its BN rows.
    // Row-major B copy i fills rows 16w + B_ROWS_PER_COPY*i + l/B_CHUNKS,
    // physical chunk l%B_CHUNKS.
    // Each operand has a uniform base (scalar registers: the tile's first row
    // of A, and the tile's first column, or first row for column-major B)
    // that a slice advances by 128 bytes of every A row (and column-major B
    // row) or by BK rows of row-major B; each copy has a 32-bit byte offset of
    // this lane's 16 bytes from it, fixed for the whole K loop.  The host
    // sends problems whose offsets do not fit in 32 bits to the masked
    // kernels (copy_offsets_fit).
    const char* a_base = reinterpret_cast<const char*>(A);
    const char* b_base = reinterpret_cast<const char*>(B);
    uint32_t a_vo[CA];
    uint32_t b_vo[CB];
    int64_t b_step = BK * ESZ;                            // bytes per slice
    uint32_t dma_a = 0, dma_b = 0;
    if constexpr (EDGE != EDGE_MASKED) {
        a_base += (int64_t)m0 * lda * ESZ;
        b_base += BT ? (int64_t)n0 * ldb * ESZ : (int64_t)n0 * ESZ;
#pragma unroll
        for (int i = 0; i < CA; ++i) {
            const int r = (BM / 4) * w + 8 * i + (l >> 3);
            int grow = m0 + r;
            if constexpr (EDGE == EDGE_CLAMP) grow = grow < M ? grow : m0 + (grow - m0) % (M - m0);
            a_vo[i] = (uint32_t)(((int64_t)(grow - m0) * lda + (16 / ESZ) * ((l & 7) ^ swz_a(r))) * ESZ);
        }
#pragma unroll
        for (int i = 0; i < CB; ++i) {
            if constexpr (BT) {
                const int r = (BN / 4) * w + 8 * i + (l >> 3);
                int gcol = n0 + r;
                if constexpr (EDGE == EDGE_CLAMP) gcol = gcol < N ? gcol : n0 + (gcol - n0) % (N - n0);
                b_vo[i] = (uint32_t)(((int64_t)(gcol - n0) * ldb + (16 / ESZ) * ((l & 7) ^ swz_a(r))) * ESZ);
            } else {
                const int kr = B_ROWS_PER_WAVE * w + B_ROWS_PER_COPY * i + l / B_CHUNKS;
                const int sw = F8 ? swz_b8<B_CHUNKS>(kr) : swz_b(kr);
                int col = n0 + (16 / ESZ) * ((l % B_CHUNKS) ^ sw);
                if constexpr (EDGE == EDGE_CLAMP) col = col + 16 / ESZ <= N ? col : n0 + (col - n0) % ((N - n0) / (16 / ESZ) * (16 / ESZ));
                b_vo[i] = (uint32_t)(((int64_t)kr * ldb + (col - n0)) * ESZ);
            }
        }
        if constexpr (!BT) b_step = (int64_t)BK * ldb * ESZ;
        dma_a = smem_base + ((BM / 4) * w) * 128;
        dma_b = smem_base + A_BYTES + (BT ? ((BN / 4) * w) * 128 : (B_ROWS_PER_WAVE * w) * BROW);
    }

    // Fragment read offsets (bytes within a stage).
    const int a_off0 = (wm * WM + (l & 31)) * 128;
    const int a_sw = swz_a(l & 31);
    const int g = l >> 4, ip = l & 15;
    const int b_sw = swz_b(ip >> 2);
    int b_off[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        if constexpr (F8 && !BT) {
            // tr8 read: lane 2jj + hh of 16-lane group G addresses row k = 32 (G / 2) + jj (+ 8 per
            // read, + 64 per k-step: the swizzle term does not change) and the 8 bytes of half hh
            // of chunk c of the lane group's 16 columns; every lane receives its own column.
            const int G = l >> 4, jj = (l & 15) >> 1, hh = l & 1;
            const int kb = 32 * (G >> 1) + jj;
            const int c = (wn * WN + 32 * j + 16 * (G & 1)) >> 4;
            b_off[j] = A_BYTES + kb * BROW + 16 * (c ^ swz_b8<B_CHUNKS>(kb)) + 8 * hh;
        } else if constexpr (BT) {
            b_off[j] = A_BYTES + (wn * WN + 32 * j + (l & 31)) * 128;
        } else {
            const int n = wn * WN + 32 * j + 16 * (g & 1) + 4 * (ip & 3);
            b_off[j] = A_BYTES + (8 * (g >> 1) + (ip >> 2)) * BROW + (((n >> 3) ^ b_sw) * 16) + (n & 7) * 2;
        }
    }

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    u32x4 fa[NB][TM];
    u32x4 fbt[NB][TN];            // column-major B fragments
    s16x4 fbh[NB][TN][2];         // row-major B fragments (two transposing reads each)
    u32x8 fa8[NB][TM], fb8[NB][TN];   // 8-bit inputs: 32 k per lane

    // LDS read q (0 .. R-1) of k-step s, in consumption order: A0, then B
    // (B0 .. B(TN-1), each as lo/hi for row-major B), then A1 .. A(TM-1).
    // 8-bit inputs: every fragment in two halves (logical chunks 4s + 2h and
    // 4s + 2h + 1 of its row, h = l / 32), in the same order.
    auto read_piece = [&](int stage, int s, int buf, int q) {
        const char* st = smem + stage * STAGE;
        if constexpr (F8) {
            if (q < RPF || q >= RPF + NBR) {                 // A fragment i, half `half`
                const int i = q < RPF ? 0 : 1 + (q - RPF - NBR) / RPF;
                const int half = q < RPF ? q : (q - RPF - NBR) % RPF;
                const int chunk = (4 * s + 2 * (l >> 5) + half) ^ a_sw;
                const u32x4 v = *reinterpret_cast<const u32x4*>(st + a_off0 + i * 32 * 128 + chunk * 16);
#pragma unroll
                for (int e = 0; e < 4; ++e) fa8[buf][i][4 * half + e] = v[e];
            } else {                                         // B fragment j, piece `piece`
                const int j = (q - RPF) / PB, piece = (q - RPF) % PB;
                if constexpr (BT) {
                    const int chunk = (4 * s + 2 * (l >> 5) + piece) ^ a_sw;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(st + b_off[j] + chunk * 16);
#pragma unroll
                    for (int e = 0; e < 4; ++e) fb8[buf][j][4 * piece + e] = v[e];
                } else {
                    const int off = b_off[j] + (64 * s + 8 * piece) * BROW;
                    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (__attribute__((address_space(3))) i32x2*)((const lds_char*)st + off));
                    fb8[buf][j][2 * piece] = (uint32_t)v[0];
                    fb8[buf][j][2 * piece + 1] = (uint32_t)v[1];
                }
            }
            return;
        }
        const int chunk = (2 * s + (l >> 5)) ^ a_sw;      // A rows and column-major B rows alike
        if (q == 0 || q > NBR) {
            const int i = (q == 0) ? 0 : q - NBR;
            fa[buf][i] = *reinterpret_cast<const u32x4*>(st + a_off0 + i * 32 * 128 + chunk * 16);
        } else if constexpr (BT) {
            const int j = q - 1;
            fbt[buf][j] = *reinterpret_cast<const u32x4*>(st + b_off[j] + chunk * 16);
        } else {
            const int j = (q - 1) >> 1, h = (q - 1) & 1;
            const int off = b_off[j] + 16 * s * BROW + h * 4 * BROW;
            fbh[buf][j][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)((const lds_char*)st + off));
        }
    };
    auto issue_copy = [&](int stage, int i) {
        if (i < 0 || i >= COPIES) return;              // never taken: callers pass 0 .. COPIES-1
        // a slice's copies are issued in index order: the bases move on after
        // the last copy of their operand
        if (i < CA) {
            lds_dma16(a_base, a_vo[i], dma_a + stage * STAGE + 1024 * i);
            if (i == CA - 1) a_base += BK * ESZ;
        } else {
            lds_dma16(b_base, b_vo[i - CA], dma_b + stage * STAGE + 1024 * (i - CA));
            if (i == COPIES - 1) b_base += b_step;
        }
    };
    // MFMA q of a k-step: A block q / TN, and B block q % TN walked
    // serpentine in the prefetch-distance-2 16-bit kernels (reversed on odd A
    // blocks), so consecutive MFMAs share an operand at every A-block change
    // too.  Each accumulator still takes its k-steps in the same order (the
    // same bits); measured +0.8% at bf16 4096^3, unchanged at 8192^3.  The
    // other kernels read their fragments in this consumption order and keep
    // the plain walk.
    auto mfma1 = [&](int buf, int q) {
        const int i = q / TN, jj = q % TN;
        const int j = (FD == 2 && !F8 && (i & 1)) ? TN - 1 - jj : jj;
        if constexpr (F8) {
            acc[i][j] = mfma8<IN>(fa8[buf][i], fb8[buf][j], acc[i][j]);
        } else if constexpr (BT) {
            acc[i][j] = mfma<IN>(fa[buf][i], fbt[buf][j], acc[i][j]);
        } else {
            const u32x2 lo = __builtin_bit_cast(u32x2, fbh[buf][j][0]);
            const u32x2 hi = __builtin_bit_cast(u32x2, fbh[buf][j][1]);
            acc[i][j] = mfma<IN>(fa[buf][i], u32x4{lo[0], lo[1], hi[0], hi[1]}, acc[i][j]);
        }
    };

    auto fill_slice = [&](int stage, int kt) {
        fill_stage<BM, BN, BT, ESZ>(smem + stage * STAGE, A, lda, B, ldb, M, N, K, m0, n0, kt * BK, t);
    };
    // One filled slice, unpipelined: the reads of each of its first `nks`
    // k-steps, then that k-step's MFMAs (the k-steps past a partial slice's
    // last valid k hold only zero fill and are skipped: adding their zero
    // products changes no sum, at most the sign of a zero).
    auto compute_slice = [&](int stage, int nks) {
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            if (s < nks) {
#pragma unroll
                for (int x = 0; x < R; ++x) read_piece(stage, s, 0, x);
#pragma unroll
                for (int q = 0; q < S; ++q) mfma1(0, q);
            }
        }
    };

    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;

    // `NS` issue slots (S or 2S): slot q runs MFMA q % S of the k-step held in
    // buffer mb[q / S], then its share of the reads of k-step rs[q / S] (into
    // buffer rb[q / S]) and, with do_copy, its share of the next slice's
    // COPIES copies.  All counts and indices are compile-time constants once
    // the calls are inlined, so every register-array index is too.
    auto block = [&](auto do_mfma, int mb0, int mb1, int rstage, int rs0, int rs1, int rb0, int rb1,
                     auto do_copy, int cstage, auto nslots_c) {
        constexpr int NS = decltype(nslots_c)::value;
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const int sub = q / S, qq = q % S;
            if constexpr (decltype(do_mfma)::value) mfma1(sub ? mb1 : mb0, qq);
#pragma unroll
            for (int x = qq * R / S; x < (qq + 1) * R / S; ++x)
                read_piece(rstage, sub ? rs1 : rs0, sub ? rb1 : rb0, x);
            if constexpr (decltype(do_copy)::value) {
#pragma unroll
                for (int c = q * COPIES / NS; c < (q + 1) * COPIES / NS; ++c) issue_copy(cstage, c);
            }
            DL_FENCE();
        }
    };

    // One slice of the pipeline over full slices: barrier (copies of slice kt
    // visible everywhere, slice kt-1 read by everyone), then the previous
    // slice's last FD k-steps with this slice's first reads and, with
    // do_copy, the copies of slice kt+1; then the remaining k-steps, each
    // interleaved with the reads FD k-steps ahead.
    auto slice = [&](int kt, auto has_prev, auto do_copy) {
        const int stage = kt & 1, nstage = stage ^ 1;
        wait_copies();                  // this wave's copies of slice kt have landed
        __syncthreads();                // everyone's; slice kt-1 is fully read
        DL_FENCE();
        using one = std::integral_constant<int, S>;
        using two = std::integral_constant<int, 2 * S>;
        if constexpr (F8) {
            // post-barrier block: previous slice's k-step 1 (buffer 1), reads of k-step 0 (buffer 0)
            block(has_prev, 1, 1, stage, 0, 0, 0, 0, do_copy, nstage, one{});
            block(yes{}, 0, 0, stage, 1, 1, 1, 1, no{}, nstage, one{});
        } else if constexpr (FD == 1) {
            // post-barrier block: previous slice's k-step 3 (buffer 1), reads of k-step 0 (buffer 0)
            block(has_prev, 1, 1, stage, 0, 0, 0, 0, do_copy, nstage, one{});
            block(yes{}, 0, 0, stage, 1, 1, 1, 1, no{}, nstage, one{});
            block(yes{}, 1, 1, stage, 2, 2, 0, 0, no{}, nstage, one{});
            block(yes{}, 0, 0, stage, 3, 3, 1, 1, no{}, nstage, one{});
        } else {
            // post-barrier block: previous slice's k-steps 2, 3 (buffers 2, 3),
            // reads of k-steps 0, 1 (buffers 0, 1)
            block(has_prev, 2, 3, stage, 0, 1, 0, 1, do_copy, nstage, two{});
            block(yes{}, 0, 0, stage, 2, 2, 2, 2, no{}, nstage, one{});
            block(yes{}, 1, 1, stage, 3, 3, 3, 3, no{}, nstage, one{});
        }
    };

    if constexpr (EDGE == EDGE_MASKED) {
        const int nk = (K + BK - 1) / BK;
        for (int kt = 0; kt < nk; ++kt) {
            __syncthreads();            // every wave is done reading the previous slice
            fill_slice(0, kt);
            __syncthreads();
            compute_slice(0, KSTEPS);
        }
    } else {
        const int nk_full = K / BK;
        if (nk_full > 0) {
#pragma unroll
            for (int i = 0; i < COPIES; ++i) issue_copy(0, i);          // slice 0 into stage 0
            if (nk_full == 1) {
                slice(0, no{}, no{});
            } else {
                slice(0, no{}, yes{});
                for (int kt = 1; kt < nk_full - 1; ++kt) slice(kt, yes{}, yes{});     // steady state
                slice(nk_full - 1, yes{}, no{});
            }
            // the last FD k-steps of the last full slice
            if constexpr (FD == 2) {
#pragma unroll
                for (int q = 0; q < S; ++q) mfma1(2, q);
#pragma unroll
                for (int q = 0; q < S; ++q) mfma1(3, q);
            } else {
#pragma unroll
                for (int q = 0; q < S; ++q) mfma1(1, q);
            }
        }
        if constexpr (EDGE == EDGE_CLAMP) {
            if (K % BK != 0) {
                // the partial last slice: zero-filled through VGPRs, then its
                // k-steps without pipelining (at most one slice in K / BK)
                const int stage = nk_full & 1;
                __syncthreads();        // every wave is done reading the stage being refilled
                fill_slice(stage, nk_full);
                __syncthreads();
                constexpr int KK = BK / KSTEPS;                      // k per k-step
                compute_slice(stage, (K % BK + KK - 1) / KK);
            }
        }
    }

    // Lane index of the epilogue's addresses.  In the edge modes it is
    // recomputed here (v_mbcnt in a volatile asm, no input), so that the
    // addresses are formed after the main loop: hoisted above a partial last
    // slice they would stay live through its VGPR fill and push accumulators
    // to scratch.
    int le = l;
    if constexpr (EDGE != EDGE_NONE)
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(le));
    const int gl = le >> 5;

    float bias_v[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        bias_v[j] = 0.0f;
        if constexpr (EPI) {
            const int col = n0 + wn * WN + 32 * j + (le & 31);
            if (ep.bias != nullptr && (EDGE == EDGE_NONE || col < N)) bias_v[j] = ep.bias[col];
        }
    }
    // The beta test and the interior test are uniform: take them once,
    // outside the element loops.  A tile wholly inside M x N stores without
    // per-element masks (a branch per element costs more than the store).
    // Edge tiles of the clamped kernels store through a buffer descriptor
    // over the tile's first element: a lane whose element lies outside M x N
    // passes an out-of-range offset, so no element needs a branch (an edge
    // tile finishes last in a one-wave launch, and per-element branches made
    // its epilogue the critical path).  The fully masked kernels, which take
    // any leading dimension, keep the branches.
    auto store_tile = [&](auto read_old, auto masked) {
        if constexpr (decltype(masked)::value && EDGE == EDGE_CLAMP) {
            constexpr int OSZ = OUT == OUT_F32 ? 4 : 2;
            const rsrc_t crs = c_rsrc(static_cast<char*>(C) + ((int64_t)m0 * ldc + n0) * OSZ);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int cl = wn * WN + 32 * j + (le & 31);            // column within the tile
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int rl = wm * WM + 32 * i + 8 * (e >> 2) + 4 * gl + (e & 3);
                        const bool ok = m0 + rl < M && n0 + cl < N;
                        const uint32_t off = ok ? ((uint32_t)rl * (uint32_t)ldc + (uint32_t)cl) * OSZ : kOutOfRange;
                        float v = acc[i][j][e];
                        if constexpr (EPI) {
                            constexpr bool ro = decltype(read_old)::value;
                            float old = 0.0f;
                            if constexpr (ro) old = load_out_buf<OUT>(crs, off);
                            v = epi_value(v, ep, ro, old, bias_v[j]);
                        }
                        store_out_buf<OUT>(crs, off, v);
                    }
                }
            }
            return;
        }
        if constexpr (ROWS && !decltype(masked)::value && TN % 2 == 0) {
            // Whole rows per store: element e of blocks j and j+1 covers rows
            // R (lanes 0-31) and R+4 (lanes 32-63) of 32 columns each; one
            // v_permlane32_swap of the two turns them into row R and row R+4
            // of all 64 columns 32j .. 32j+63, so every store instruction
            // writes 64 consecutive elements of one row (128 bytes of a
            // 16-bit output, whole cache lines when the rows are aligned)
            // instead of two 32-element pieces.  Four elements at a time.
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int j = 0; j < TN; j += 2) {
                    const int col = n0 + wn * WN + 32 * j + le;
                    const float bias_c = le < 32 ? bias_v[j] : bias_v[j + 1];
#pragma unroll
                    for (int e0 = 0; e0 < 16; e0 += 4) {
                        uint32_t x[4], y[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            // through a float: a bit cast taken straight from
                            // the vector subscript read the same register for
                            // every subscript
                            const float xa = acc[i][j][e0 + q], ya = acc[i][j + 1][e0 + q];
                            x[q] = __float_as_uint(xa);
                            y[q] = __float_as_uint(ya);
                        }
                        permlane32_swap4(x[0], y[0], x[1], y[1], x[2], y[2], x[3], y[3]);
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int e = e0 + (q >> 1), h = q & 1;     // h: row R or R+4
                            const int row = m0 + wm * WM + 32 * i + 8 * (e >> 2) + (e & 3) + 4 * h;
                            const int64_t idx = (int64_t)row * ldc + col;
                            float v = __uint_as_float(h ? y[q >> 1] : x[q >> 1]);
                            if constexpr (EPI) {
                                constexpr bool ro = decltype(read_old)::value;
                                float old = 0.0f;
                                if constexpr (ro) old = load_out<OUT>(C, idx);
                                v = epi_value(v, ep, ro, old, bias_c);
                            }
                            store_out<OUT, NTC>(C, idx, v);
                        }
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int col = n0 + wn * WN + 32 * j + (le & 31);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = m0 + wm * WM + 32 * i + 8 * (e >> 2) + 4 * gl + (e & 3);
                    if (!decltype(masked)::value || (row < M && col < N)) {
                        const int64_t idx = (int64_t)row * ldc + col;
                        float v = acc[i][j][e];
                        if constexpr (EPI) {
                            constexpr bool ro = decltype(read_old)::value;
                            float old = 0.0f;
                            if constexpr (ro) old = load_out<OUT>(C, idx);
                            v = epi_value(v, ep, ro, old, bias_v[j]);
                        }
                        store_out<OUT, NTC>(C, idx, v);
                    }
                }
            }
        }
    };
    auto store_edge = [&](auto read_old) {
        if constexpr (EDGE == EDGE_NONE) {
            store_tile(read_old, no{});
        } else {
            if (m0 + BM <= M && n0 + BN <= N)
                store_tile(read_old, no{});
            else
                store_tile(read_old, yes{});
        }
    };
    if (EPI && ep.beta != 0.0f)
        store_edge(yes{});
    else
        store_edge(no{});
}

// One workgroup per output tile, tiles in the tile_coords order.
template <int IN, int OUT, int BM, int BN, int FD, int EDGE, bool BT, bool EPI>
__global__ __launch_bounds__(256, 1) void gemm_dl_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tilesM, int tilesN, int group_m,
    EpiArgs ep) {
#ifdef DHPT_TIMELINE
    const TlStamp tl0 = tl_now();
#endif
    __shared__ __attribute__((aligned(1024))) char smem[dl_lds_bytes<IN, BM, BN, EDGE, BT>()];
    int tm, tn;
    tile_coords(blockIdx.x, tilesM, tilesN, group_m, &tm, &tn);
    constexpr bool NTC = EDGE == EDGE_NONE;          // non-temporal C stores on whole tiles
    dl_tile<IN, OUT, BM, BN, FD, EDGE, BT, EPI, NTC, true>(smem, A, lda, B, ldb, C, ldc, M, N, K, tm * BM, tn * BN,
                                                           ep, (int)threadIdx.x);
#ifdef DHPT_TIMELINE
    tl_record(ep.timeline, tl0);
#endif
}

// The persistent form: a grid of at most one workgroup per CU, each taking
// tiles from shared counters until none is left -- the persistent kernel of
// "The Asynchronous Kernel: Tensor Cores & TMA" (section "Keeping the line
// busy"), with one queue per XCD.  Queue x holds the logical ids
// [xcd_first(x), xcd_first(x + 1)) that the one-workgroup-per-tile launch
// deals to XCD x, in the same order, so each XCD's L2 sees the same compact
// block of the grouped order; a workgroup takes from the queue of the XCD it
// runs on (read from the hardware register) and, once that is empty, from the
// other queues in turn, so the XCDs that run ahead (they hold different
// clocks) take over the last tiles of the slow ones.  A tile index comes from
// a vector-memory atomic add at device scope on the queue's head; the index
// of the next tile is fetched while the current one is computed.  There are
// no waits between workgroups: a workgroup that finds every queue drained
// exits, and the last one to exit (counted by a second atomic) resets the
// heads to zero for the next launch.
//
// Scheduler words (uint32) in the caller's workspace: the head of XCD x's
// queue at kSchedStride * x (one 256-byte line each), the count of finished
// workgroups at kSchedDone.  They must be zero when the kernel starts; the
// kernel leaves them zero when it ends.
constexpr int kSchedStride = 64;
constexpr int kSchedDone = 8 * kSchedStride;
constexpr int kSchedBytes = 4 * (kSchedDone + kSchedStride);

__device__ __forceinline__ int sched_pull(uint32_t* sched, int xcd, int T) {
    for (int d = 0; d < 8; ++d) {
        const int x = (xcd + d) & 7;
        const int first = xcd_first(x, T), cnt = xcd_first(x + 1, T) - first;
        if (cnt == 0) continue;
        const uint32_t h =
            __hip_atomic_fetch_add(sched + kSchedStride * x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (h < (uint32_t)cnt) return first + (int)h;
    }
    return -1;
}

template <int IN, int OUT, int BM, int BN, int FD, int EDGE, bool BT, bool EPI>
__global__ __launch_bounds__(256, 1) void gemm_dl_persist_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, int M, int N, int K, int tilesM, int tilesN, int group_m,
    EpiArgs ep, uint32_t* __restrict__ sched) {
#ifdef DHPT_TIMELINE
    const TlStamp tl0 = tl_now();
#endif
    __shared__ __attribute__((aligned(1024))) char smem[dl_lds_bytes<IN, BM, BN, EDGE, BT>()];
    __shared__ int next_tile;
    const int T = tilesM * tilesN;
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const int xcd = (int)(xcc & 7);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);     // kept in a scalar register
    if (threadIdx.x == 0) next_tile = sched_pull(sched, xcd, T);
    __syncthreads();
    int L = __builtin_amdgcn_readfirstlane(next_tile);
#ifdef DHPT_TIMELINE
    uint32_t tiles_done = 0;
#endif
    while (L >= 0) {
#ifdef DHPT_TIMELINE
        ++tiles_done;
#endif
        __syncthreads();                    // every lane has read next_tile
        if (threadIdx.x == 0) next_tile = sched_pull(sched, xcd, T);
        int tm, tn;
        grouped_tile(L, tilesM, tilesN, group_m, &tm, &tn);
        // threadIdx.x rebuilt per tile from the wave index and the lane
        // index (v_mbcnt in a volatile asm): nothing per lane stays live
        // across the tile loop
        int lane;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
        const int tid = 64 * wave + lane;
        constexpr bool NTC = EDGE == EDGE_NONE;      // non-temporal C stores on whole tiles
        dl_tile<IN, OUT, BM, BN, FD, EDGE, BT, EPI, NTC>(smem, A, lda, B, ldb, C, ldc, M, N, K, tm * BM, tn * BN, ep,
                                                         tid);
        __syncthreads();                    // the stages are free; next_tile is published
        L = __builtin_amdgcn_readfirstlane(next_tile);
    }
    if (threadIdx.x == 0) {
        // Every pull of this workgroup has returned; the last workgroup to get
        // here knows that every pull of the launch has, and resets the heads.
        const uint32_t done =
            __hip_atomic_fetch_add(sched + kSchedDone, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            for (int x = 0; x < 8; ++x)
                __hip_atomic_store(sched + kSchedStride * x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sched + kSchedDone, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
#ifdef DHPT_TIMELINE
    tl_record(ep.timeline, tl0, tiles_done);
#endif
}

template <int IN, int OUT, int BM, int BN, int FD, int EDGE, bool BT, bool EPI>
static void launch_persist_typed(const Problem& p, int group_m, hipStream_t s) {
    const int tilesM = (p.M + BM - 1) / BM, tilesN = (p.N + BN - 1) / BN;
    const int T = tilesM * tilesN;
    const int grid = T < p.workers ? T : p.workers;
    EpiArgs ep{p.alpha, p.beta, p.bias, p.relu};
#ifdef DHPT_TIMELINE
    ep.timeline = timeline_for((int64_t)grid * 4);
#endif
    hipLaunchKernelGGL((gemm_dl_persist_kernel<IN, OUT, BM, BN, FD, EDGE, BT, EPI>), dim3((unsigned)grid), dim3(256), 0,
                       s, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.M, p.N, p.K, tilesM, tilesN, group_m, ep, p.sched);
}

// The persistent 256x256 kernels for 16-bit inputs (EDGE_NONE, EDGE_CLAMP).
template <bool BT, bool EPI>
static hipError_t launch_persist_family(int edge, const Problem& p, int group_m, hipStream_t s) {
    if (edge != EDGE_NONE && edge != EDGE_CLAMP) return hipErrorInvalidValue;
    auto go = [&](auto edge_c) {
        constexpr int E = decltype(edge_c)::value;
        switch (p.dtype) {
        case 0: launch_persist_typed<IN_F16, OUT_F32, 256, 256, 2, E, BT, EPI>(p, group_m, s); break;
        case 1: launch_persist_typed<IN_F16, OUT_F16, 256, 256, 2, E, BT, EPI>(p, group_m, s); break;
        case 2: launch_persist_typed<IN_BF16, OUT_F32, 256, 256, 2, E, BT, EPI>(p, group_m, s); break;
        case 3: launch_persist_typed<IN_BF16, OUT_BF16, 256, 256, 2, E, BT, EPI>(p, group_m, s); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    };
    return edge == EDGE_NONE ? go(std::integral_constant<int, EDGE_NONE>{})
                             : go(std::integral_constant<int, EDGE_CLAMP>{});
}

template <int IN, int OUT, int BM, int BN, int FD, int EDGE, bool BT, bool EPI>
static void launch_typed(const Problem& p, int group_m, hipStream_t s) {
    const int tilesM = (p.M + BM - 1) / BM, tilesN = (p.N + BN - 1) / BN;
    EpiArgs ep{p.alpha, p.beta, p.bias, p.relu};
#ifdef DHPT_TIMELINE
    ep.timeline = timeline_for((int64_t)tilesM * tilesN * 4);
#endif
    hipLaunchKernelGGL((gemm_dl_kernel<IN, OUT, BM, BN, FD, EDGE, BT, EPI>), dim3((unsigned)(tilesM * tilesN)),
                       dim3(256), 0, s, p.A, p.lda, p.B, p.ldb, p.C, p.ldc, p.M, p.N, p.K, tilesM, tilesN,
                       group_m, ep);
}

template <int BM, int BN, int FD, int EDGE, bool BT, bool EPI>
static hipError_t launch_dtype(const Problem& p, int group_m, hipStream_t s) {
    switch (p.dtype) {
    case 0: launch_typed<IN_F16, OUT_F32, BM, BN, FD, EDGE, BT, EPI>(p, group_m, s); break;
    case 1: launch_typed<IN_F16, OUT_F16, BM, BN, FD, EDGE, BT, EPI>(p, group_m, s); break;
    case 2: launch_typed<IN_BF16, OUT_F32, BM, BN, FD, EDGE, BT, EPI>(p, group_m, s); break;
    case 3: launch_typed<IN_BF16, OUT_BF16, BM, BN, FD, EDGE, BT, EPI>(p, group_m, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// The 8-bit input dtypes (4 .. 9: E4M3 then E5M2, each to fp32, fp16, bf16).
template <int BM, int BN, int EDGE, bool BT, bool EPI>
static hipError_t launch_dtype8(const Problem& p, int group_m, hipStream_t s) {
    switch (p.dtype) {
    case 4: launch_typed<IN_E4M3, OUT_F32, BM, BN, 1, EDGE, BT, EPI>(p, group_m, s); break;
    case 5: launch_typed<IN_E4M3, OUT_F16, BM, BN, 1, EDGE, BT, EPI>(p, group_m, s); break;
    case 6: launch_typed<IN_E4M3, OUT_BF16, BM, BN, 1, EDGE, BT, EPI>(p, group_m, s); break;
    case 7: launch_typed<IN_E5M2, OUT_F32, BM, BN, 1, EDGE, BT, EPI>(p, group_m, s); break;
    case 8: launch_typed<IN_E5M2, OUT_F16, BM, BN, 1, EDGE, BT, EPI>(p, group_m, s); break;
    case 9: launch_typed<IN_E5M2, OUT_BF16, BM, BN, 1, EDGE, BT, EPI>(p, group_m, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// All tile sizes and edge modes for 8-bit inputs and one B layout.  Clamped
// edges cover every shape for column-major B and N % 16 == 0 for row-major
// B; the masked mode (256 and 128 tiles) takes any shape and any leading
// dimension.
template <bool BT, bool EPI>
static hipError_t launch_family8(int tile, int edge, const Problem& p, int group_m, hipStream_t s) {
    if (edge == EDGE_MASKED)
        return tile == 256 ? launch_dtype8<256, 256, EDGE_MASKED, BT, EPI>(p, group_m, s)
                           : launch_dtype8<128, 128, EDGE_MASKED, BT, EPI>(p, group_m, s);
    if (tile == 256)
        return edge == EDGE_NONE ? launch_dtype8<256, 256, EDGE_NONE, BT, EPI>(p, group_m, s)
                                 : launch_dtype8<256, 256, EDGE_CLAMP, BT, EPI>(p, group_m, s);
    if (tile == 128)
        return edge == EDGE_NONE ? launch_dtype8<128, 128, EDGE_NONE, BT, EPI>(p, group_m, s)
                                 : launch_dtype8<128, 128, EDGE_CLAMP, BT, EPI>(p, group_m, s);
    return edge == EDGE_NONE ? launch_dtype8<64, 64, EDGE_NONE, BT, EPI>(p, group_m, s)
                             : launch_dtype8<64, 64, EDGE_CLAMP, BT, EPI>(p, group_m, s);
}

// All tile sizes and edge modes for one (FD, BT, EPI) combination.  The
// masked mode does not pipeline, so it exists only once, under FD == 2.
template <int FD, bool BT, bool EPI>
static hipError_t launch_family(int tile, int edge, const Problem& p, int group_m, hipStream_t s) {
    if (edge == EDGE_MASKED) {
        if constexpr (FD == 2) {
            return tile == 256 ? launch_dtype<256, 256, 2, EDGE_MASKED, BT, EPI>(p, group_m, s)
                               : launch_dtype<128, 128, 2, EDGE_MASKED, BT, EPI>(p, group_m, s);
        } else {
            return hipErrorInvalidValue;
        }
    }
    if (tile == 256)
        return edge == EDGE_NONE ? launch_dtype<256, 256, FD, EDGE_NONE, BT, EPI>(p, group_m, s)
                                 : launch_dtype<256, 256, FD, EDGE_CLAMP, BT, EPI>(p, group_m, s);
    if (tile == 64) {
        if constexpr (FD == 2) {
            return edge == EDGE_NONE ? launch_dtype<64, 64, 2, EDGE_NONE, BT, EPI>(p, group_m, s)
                                     : launch_dtype<64, 64, 2, EDGE_CLAMP, BT, EPI>(p, group_m, s);
        } else {
            return hipErrorInvalidValue;
        }
    }
    return edge == EDGE_NONE ? launch_dtype<128, 128, FD, EDGE_NONE, BT, EPI>(p, group_m, s)
                             : launch_dtype<128, 128, FD, EDGE_CLAMP, BT, EPI>(p, group_m, s);
}

}  // namespace dl
}  // namespace dhpt
