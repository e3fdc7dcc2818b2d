// gemm_common.h -- device helpers shared by the gfx950 GEMM kernel templates
// (gemm_dl_kernel.h, gemm_ks_kernel.h): operand types, the MFMAs and output
// conversions, the LDS swizzles, the asynchronous global -> LDS copy, and the
// zero-filling slice fill through VGPRs used at ragged edges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_internal.h"

namespace dhpt {
namespace dl {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

// Input formats: fp16 and bf16 (2-byte elements), and the 8-bit floats E4M3
// and E5M2 of the OCP 8-bit floating point specification (1-byte elements).
enum { IN_F16 = 0, IN_BF16 = 1, IN_E4M3 = 2, IN_E5M2 = 3 };
template <int IN>
constexpr bool kIn8 = IN == IN_E4M3 || IN == IN_E5M2;
enum { OUT_F32 = 0, OUT_F16 = 1, OUT_BF16 = 2 };
enum { EDGE_NONE = 0, EDGE_CLAMP = 1, EDGE_MASKED = 2 };

template <int IN>
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (IN == IN_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x64_f8f6f4 with A and B in one 8-bit format: lane l holds
// row (A) or column (B) l % 32 and 32 values of k, the same 32 for A and B
// (the probe tests pin that the two operands share their k assignment, and
// that format codes 0 and 1 read E4M3 and E5M2).  The scale operands are 0,
// which selects the unscaled instruction.
template <int IN>
__device__ __forceinline__ f32x16 mfma8(u32x8 a, u32x8 b, f32x16 c) {
    constexpr int fmt = IN == IN_E4M3 ? 0 : 1;
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                            __builtin_bit_cast(i32x8, b), c, fmt, fmt,
                                                            0, 0, 0, 0);
}

// NT: a non-temporal store (the `nt` cache policy), for output that no later
// step of the same kernel reads: it does not take L2 lines from the operand
// panels still being streamed, and the end of the kernel has fewer dirty
// lines to write back.  The value stored is the same either way.
template <int OUT, bool NT = false>
__device__ __forceinline__ void store_out(void* C, int64_t idx, float v) {
    if constexpr (NT) {
        if constexpr (OUT == OUT_F32)
            __builtin_nontemporal_store(v, static_cast<float*>(C) + idx);
        else if constexpr (OUT == OUT_F16)
            __builtin_nontemporal_store((_Float16)v, static_cast<_Float16*>(C) + idx);
        else
            __builtin_nontemporal_store(__builtin_bit_cast(unsigned short, (__bf16)v),
                                        static_cast<unsigned short*>(C) + idx);
    } else if constexpr (OUT == OUT_F32) {
        static_cast<float*>(C)[idx] = v;
    } else if constexpr (OUT == OUT_F16) {
        static_cast<_Float16*>(C)[idx] = (_Float16)v;     // v_cvt_f16_f32: round to nearest even
    } else {
        static_cast<__bf16*>(C)[idx] = (__bf16)v;         // round to nearest even
    }
}

template <int OUT>
__device__ __forceinline__ float load_out(const void* C, int64_t idx) {
    if constexpr (OUT == OUT_F32)
        return static_cast<const float*>(C)[idx];
    else if constexpr (OUT == OUT_F16)
        return (float)static_cast<const _Float16*>(C)[idx];
    else
        return (float)static_cast<const __bf16*>(C)[idx];
}

__device__ __forceinline__ int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz_b(int k) { return 2 * (k & 3); }
// Row-major 8-bit B, CPR 16-byte chunks per row: chunk c of row k sits at
// c ^ swz_b8<CPR>(k).  A ds_read_b64_tr_b8 pass (32 lanes) reads chunks c, c+1
// (c even) of 8 consecutive rows; the XOR puts those 16 chunks on 16
// different groups of 4 banks for every row length used (256, 128, 64 bytes).
template <int CPR>
__device__ __forceinline__ int swz_b8(int k) {
    constexpr int R = CPR < 16 ? 16 / CPR : 1;  // rows per 64-bank cycle
    return 2 * ((k / R) & (CPR / 2 - 1));
}

// One global_load_lds_dwordx4 (this lane's 16 bytes at sbase + voff to LDS
// byte address lds_base + 16 * lane), issued through inline assembly so that
// the compiler does not make every later LDS read wait for it; its completion
// is awaited explicitly (vmcnt) before the barrier that publishes the stage.
// The scalar-base form: sbase is uniform (a scalar register pair) and voff a
// byte offset below 2^31, so a copy reads one address VGPR instead of two, and a
// slice advances two scalar bases instead of every lane's 64-bit pointers
// (measured 2-3% faster on the 256x256 kernels than 64-bit lane addresses).
// M0 has no other user in this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

// v_permlane32_swap_b32 on four pairs: in each, lanes 32-63 of x trade
// places with lanes 0-31 of y (x becomes {x[0..31], y[0..31]}, y becomes
// {x[32..63], y[32..63]}; pinned by a probe test).  The instruction needs two
// wait states after a VALU write of its operands; assembly gets none from the
// compiler, hence the s_nop 1 before the group (each later swap of the group
// is further from those writes) and, conservatively, one after it.  Four to
// a group, in assembly: the builtin, one swap at a time, pushed the 256x256
// epilogue into scratch.
__device__ __forceinline__ void permlane32_swap4(uint32_t& x0, uint32_t& y0, uint32_t& x1, uint32_t& y1,
                                                 uint32_t& x2, uint32_t& y2, uint32_t& x3, uint32_t& y3) {
    asm volatile("s_nop 1\n\t"
                 "v_permlane32_swap_b32 %0, %1\n\t"
                 "v_permlane32_swap_b32 %2, %3\n\t"
                 "v_permlane32_swap_b32 %4, %5\n\t"
                 "v_permlane32_swap_b32 %6, %7\n\t"
                 "s_nop 1"
                 : "+v"(x0), "+v"(y0), "+v"(x1), "+v"(y1), "+v"(x2), "+v"(y2), "+v"(x3), "+v"(y3));
}

__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

#define DL_FENCE() __builtin_amdgcn_sched_barrier(0)

// Element type of an operand's bit patterns: uint16_t for the 16-bit
// formats, uint8_t for the 8-bit ones.
template <int ESZ>
using elem_t = std::conditional_t<ESZ == 2, uint16_t, uint8_t>;

// One 16-byte chunk of a row of ESZ-byte elements: CH = 16 / ESZ consecutive
// values p[c0 .. c0+CH-1] of the row p[0 .. limit-1], those at index >= limit
// reading as zero.  Element loads: any limit >= 1.
template <int ESZ>
__device__ __forceinline__ u32x4 load_chunk_masked(const elem_t<ESZ>* p, int c0, int limit) {
    constexpr int CH = 16 / ESZ;
    if (c0 + CH <= limit) return *reinterpret_cast<const u32x4*>(p + c0);
    uint32_t h[CH];
#pragma unroll
    for (int e = 0; e < CH; ++e) h[e] = (c0 + e < limit) ? (uint32_t)p[c0 + e] : 0u;
    if constexpr (ESZ == 2)
        return u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    else
        return u32x4{h[0] | (h[1] << 8) | (h[2] << 16) | (h[3] << 24), h[4] | (h[5] << 8) | (h[6] << 16) | (h[7] << 24),
                     h[8] | (h[9] << 8) | (h[10] << 16) | (h[11] << 24),
                     h[12] | (h[13] << 8) | (h[14] << 16) | (h[15] << 24)};
}

// The same for limit >= CH, without a branch, in two steps so that a caller
// can issue every load of a fill before the first shift: load_chunk_at reads
// the last whole in-row chunk at or before c0, shift_chunk moves the wanted
// values down by the distance (CH or more clears the chunk).
template <int ESZ>
__device__ __forceinline__ u32x4 load_chunk_at(const elem_t<ESZ>* p, int c0, int limit, int* sh) {
    constexpr int CH = 16 / ESZ;
    const int start = c0 < limit - CH ? c0 : limit - CH;    // [start, start + CH) lies in the row
    const int d = c0 - start;                               // 0 whole, 1..CH-1 partial, >= CH past the end
    *sh = d < CH ? d : CH;
    return *reinterpret_cast<const u32x4*>(p + start);
}
template <int ESZ>
__device__ __forceinline__ u32x4 shift_chunk(u32x4 v, int sh) {
    unsigned __int128 x = __builtin_bit_cast(unsigned __int128, v);
    x = (x >> (4 * ESZ * sh)) >> (4 * ESZ * sh);            // two shifts of <= 64 bits: CH clears all
    return __builtin_bit_cast(u32x4, x);
}

// Raw buffer access to C for edge tiles: a descriptor over the tile's first
// element with 2^31 bytes of range, so that a lane whose element lies outside
// M x N passes the offset kOutOfRange instead of branching around its access:
// the hardware drops such a store and returns zero for such a load.  The
// host keeps every in-range offset below 2^31 (c_offsets_fit).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ rsrc_t c_rsrc(void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)kOutOfRange, 0x00020000);
}

template <int OUT>
__device__ __forceinline__ void store_out_buf(rsrc_t r, uint32_t off, float v) {
    if constexpr (OUT == OUT_F32)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
    else if constexpr (OUT == OUT_F16)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (_Float16)v), r, off, 0, 0);
    else
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), r, off, 0, 0);
}

template <int OUT>
__device__ __forceinline__ float load_out_buf(rsrc_t r, uint32_t off) {
    if constexpr (OUT == OUT_F32)
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    else if constexpr (OUT == OUT_F16)
        return (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
    else
        return (float)__builtin_bit_cast(__bf16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}

// The epilogue operands of the general form (unused by the plain kernels).
// Profiling builds (-DDHPT_TIMELINE, a separate library) also carry the
// timeline buffer through it.
struct EpiArgs {
    float alpha, beta;
    const float* bias;         // N values, or null
    int relu;
#ifdef DHPT_TIMELINE
    uint64_t* timeline;        // 8 words per wave, or null
#endif
};

#ifdef DHPT_TIMELINE
// Profiling builds only.  A timestamp: the constant-rate real-time counter
// (s_memrealtime, 100 MHz) and the shader-clock counter (s_memtime).
struct TlStamp {
    uint64_t real, clk;
};
__device__ __forceinline__ TlStamp tl_now() {
    return TlStamp{__builtin_amdgcn_s_memrealtime(), __builtin_amdgcn_s_memtime()};
}
// Called last by every wave: once the wave's stores have completed, lane 0
// writes {start, end (real time), start, end (shader clock), XCC id << 32 |
// HW_ID, workgroup id, tiles, 0} to record blockIdx.x * waves + wave of
// `buf` (8 words per record; `tiles`: output tiles the workgroup computed).
__device__ __forceinline__ void tl_record(uint64_t* buf, TlStamp t0, uint32_t tiles = 1) {
    if (buf == nullptr) return;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const TlStamp t1 = tl_now();
    uint32_t hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if ((threadIdx.x & 63) == 0) {
        uint64_t* r = buf + 8 * ((uint64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
        r[0] = t0.real;
        r[1] = t1.real;
        r[2] = t0.clk;
        r[3] = t1.clk;
        r[4] = ((uint64_t)xcc << 32) | hw;
        r[5] = blockIdx.x;
        r[6] = tiles;
    }
}
#endif

// The general epilogue's fp32 value, in one fixed order: alpha * acc
// (rounded), plus beta * C_old in one fused step when C_old is read, plus the
// bias (rounded), then ReLU.  Contraction is off, so every instantiation
// (every output type) computes this same value before its one rounding.
__device__ __forceinline__ float epi_value(float acc, const EpiArgs& ep, bool read_old, float old, float bias) {
#pragma clang fp contract(off)
    float v = ep.alpha * acc;
    if (read_old) v = fmaf(ep.beta, old, v);
    v = v + bias;
    return (ep.relu && v < 0.0f) ? 0.0f : v;
}

// One slice (128 bytes of every row: k0 .. k0+63 for 2-byte elements,
// k0 .. k0+127 for 1-byte ones) of the A rows m0 .. m0+BM-1 and of B (columns
// n0 .. n0+BN-1) into the LDS stage `st` through VGPRs, with every value
// outside M x K (A) and K x N (B) read as zero, in the stage layout of the
// direct-to-LDS copies: A BM rows x 128 bytes, chunk c of row r at
// c ^ swz_a(r); row-major B 128/ESZ rows x ESZ*BN bytes, chunk c of row k at
// c ^ swz_b(k) (2-byte elements) or c ^ swz_b8(k) (1-byte); column-major B BN
// rows x 128 bytes like A.  All 256 lanes of the workgroup take part.  All
// loads are issued before the first LDS write: rows past the edge read a
// clamped valid row and are zeroed afterwards, and chunks crossing the row
// end use the branch-free shifted load whenever the row holds at least one
// chunk of values (a uniform test), so one memory round trip fills the slice.
// ESZ is the element size in bytes.
template <int BM, int BN, bool BT, int ESZ = 2>
__device__ __forceinline__ void fill_stage(char* st, const uint16_t* A, int64_t lda,
                                           const uint16_t* B, int64_t ldb, int M, int N,
                                           int K, int m0, int n0, int k0, int t) {
    constexpr int CH = 16 / ESZ;                                  // elements per 16-byte chunk
    constexpr int BKR = 128 / ESZ;                                // k (B rows) per slice
    constexpr int A_BYTES = BM * 128, BROW = ESZ * BN, B_CHUNKS = BROW / 16;
    constexpr int NFA = BM / 32;                                  // A chunks per lane
    constexpr int B_ROWS_PER_PASS = 256 / B_CHUNKS;
    constexpr int NFB = BT ? BN / 32 : BKR / B_ROWS_PER_PASS;     // B chunks per lane
    using E = elem_t<ESZ>;
    const E* const Ae = reinterpret_cast<const E*>(A);
    const E* const Be = reinterpret_cast<const E*>(B);
    const u32x4 zero = u32x4{0u, 0u, 0u, 0u};
    u32x4 va[NFA], vb[NFB];
    const E* pa[NFA];
    const E* pb[NFB];
    int cb[NFB];
#pragma unroll
    for (int r = 0; r < NFA; ++r) {                // A: BM rows x 8 chunks
        const int grow = m0 + (t >> 3) + 32 * r;
        pa[r] = Ae + (int64_t)(grow < M ? grow : M - 1) * lda;
    }
#pragma unroll
    for (int r = 0; r < NFB; ++r) {
        if constexpr (BT) {                        // column-major B: BN rows x 8 chunks
            const int gcol = n0 + (t >> 3) + 32 * r;
            pb[r] = Be + (int64_t)(gcol < N ? gcol : N - 1) * ldb;
            cb[r] = k0 + CH * (t & 7);
        } else {                                   // row-major B: 64 rows x B_CHUNKS chunks
            const int gk = k0 + t / B_CHUNKS + B_ROWS_PER_PASS * r;
            pb[r] = Be + (int64_t)(gk < K ? gk : K - 1) * ldb;
            cb[r] = n0 + CH * (t % B_CHUNKS);
        }
    }
    const int ca = k0 + CH * (t & 7);
    const int blim = BT ? K : N;                   // valid length of a B row
    if (K >= CH && blim >= CH) {                   // every load in flight before the first shift
        int sha[NFA], shb[NFB];
#pragma unroll
        for (int r = 0; r < NFA; ++r) va[r] = load_chunk_at<ESZ>(pa[r], ca, K, &sha[r]);
#pragma unroll
        for (int r = 0; r < NFB; ++r) vb[r] = load_chunk_at<ESZ>(pb[r], cb[r], blim, &shb[r]);
        DL_FENCE();
#pragma unroll
        for (int r = 0; r < NFA; ++r) va[r] = shift_chunk<ESZ>(va[r], sha[r]);
#pragma unroll
        for (int r = 0; r < NFB; ++r) vb[r] = shift_chunk<ESZ>(vb[r], shb[r]);
    } else {
#pragma unroll
        for (int r = 0; r < NFA; ++r) va[r] = load_chunk_masked<ESZ>(pa[r], ca, K);
#pragma unroll
        for (int r = 0; r < NFB; ++r) vb[r] = load_chunk_masked<ESZ>(pb[r], cb[r], blim);
    }
#pragma unroll
    for (int r = 0; r < NFA; ++r) {
        const int row = (t >> 3) + 32 * r, c = t & 7;
        *reinterpret_cast<u32x4*>(st + row * 128 + 16 * (c ^ swz_a(row))) = m0 + row < M ? va[r] : zero;
    }
#pragma unroll
    for (int r = 0; r < NFB; ++r) {
        if constexpr (BT) {
            const int row = (t >> 3) + 32 * r, c = t & 7;
            *reinterpret_cast<u32x4*>(st + A_BYTES + row * 128 + 16 * (c ^ swz_a(row))) =
                n0 + row < N ? vb[r] : zero;
        } else {
            const int row = t / B_CHUNKS + B_ROWS_PER_PASS * r, c = t % B_CHUNKS;
            if constexpr (ESZ == 2)
                *reinterpret_cast<u32x4*>(st + A_BYTES + row * BROW + 16 * (c ^ swz_b(row))) =
                    k0 + row < K ? vb[r] : zero;
            else
                *reinterpret_cast<u32x4*>(st + A_BYTES + row * BROW + 16 * (c ^ swz_b8<B_CHUNKS>(row))) =
                    k0 + row < K ? vb[r] : zero;
        }
    }
}

}  // namespace dl
}  // namespace dhpt
