// bench_probe.hip -- the MFMA-only reference loop that bench.py times beside
// the GEMM (built into libdhpt_bench_probe.so next to this file).
//
// Every wave (4 per workgroup, one per SIMD; one workgroup per CU at the
// launch sizes used) keeps eight independent 32x32 accumulators and issues
// MFMAs back to back, with no memory traffic inside the loop.  The operands
// are the same kind of data the GEMM workloads multiply (bf16 N(0,1), fp16
// U[-1,1), E4M3 N(0,1)), loaded once and rotated so that consecutive MFMAs
// see different values, as they do in a GEMM: the clock the chip holds under
// MFMAs depends on the operand bits, so a constant-operand loop would
// overstate what the GEMM can reach.  Its rate is the practical MFMA ceiling
// for that data, the denominator of the "probe peak" fraction; counting the
// instructions at the observed clock gives the FLOP/clk/CU figure that the
// Ada tensor-core GEMM write-up asks for when benchmarking matrix units
// (measure the rate at the clock actually held, against the nominal one).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

enum { FMT_F16 = 0, FMT_BF16 = 1, FMT_E4M3 = 2 };

// ops: for 16-bit formats 16 x 64 lanes x 16 bytes (a and b fragments 0..7
// interleaved); for E4M3 32 x 64 lanes x 16 bytes (two 16-byte halves per
// 32-byte fragment).  Each iteration issues 32 MFMAs per wave.
template <int FMT>
__global__ __launch_bounds__(256, 1) void mfma_loop_kernel(const u32x4* __restrict__ ops, int iters,
                                                           float* __restrict__ sink, uint64_t* __restrict__ clocks) {
    const uint64_t real0 = __builtin_amdgcn_s_memrealtime(), clk0 = __builtin_amdgcn_s_memtime();
    const int l = threadIdx.x & 63;
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (f32x16){};
    if constexpr (FMT == FMT_E4M3) {
        i32x8 a[8], b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const u32x4 a0 = ops[(4 * i) * 64 + l], a1 = ops[(4 * i + 1) * 64 + l];
            const u32x4 b0 = ops[(4 * i + 2) * 64 + l], b1 = ops[(4 * i + 3) * 64 + l];
            a[i] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2],
                         (int)a1[3]};
            b[i] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2],
                         (int)b1[3]};
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(i + r) & 7], b[(i + 3 * r) & 7],
                                                                             acc[i], 0, 0, 0, 0, 0, 0);
        }
    } else {
        u32x4 a[8], b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = ops[(2 * i) * 64 + l];
            b[i] = ops[(2 * i + 1) * 64 + l];
        }
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const u32x4 av = a[(i + r) & 7], bv = b[(i + 3 * r) & 7];
                    if constexpr (FMT == FMT_BF16)
                        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                                         __builtin_bit_cast(bf16x8, bv), acc[i], 0, 0, 0);
                    else
                        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                                        __builtin_bit_cast(f16x8, bv), acc[i], 0, 0, 0);
                }
        }
    }
    // keep the accumulators live; the sum is never the sentinel in practice
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
    if (s == 12345.0f) sink[0] = s;
    // the wave's run time on the 100 MHz real-time counter and on the shader
    // clock (s_memtime), for the clock the loop ran at
    if (clocks != nullptr && l == 0) {
        const uint64_t real1 = __builtin_amdgcn_s_memrealtime(), clk1 = __builtin_amdgcn_s_memtime();
        const uint64_t i = 2 * ((uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6));
        clocks[i] = real1 - real0;
        clocks[i + 1] = clk1 - clk0;
    }
}

}  // namespace

extern "C" {

// Enqueue the loop on `stream` (a hipStream_t; NULL = the null stream):
// `blocks` workgroups of 256 lanes, `iters` x 32 MFMAs per wave.  fmt 0 fp16,
// 1 bf16 (v_mfma_f32_32x32x16, 32768 FLOP each), 2 E4M3
// (v_mfma_f32_32x32x64_f8f6f4, 131072 FLOP each).  ops: device buffer of
// ops_bytes bytes, at least 16 KiB (16-bit formats) or 32 KiB (E4M3), 16-byte
// aligned; sink: one device float; clocks: null, or 2 x 4 x blocks uint64
// that receive per wave the run time in 10 ns ticks and in shader clocks.
// Returns 0, or -1 for bad arguments (an undersized buffer included), or the
// HIP error of the launch.
int bench_probe_mfma(int fmt, int blocks, int iters, const void* ops, int64_t ops_bytes, float* sink,
                     uint64_t* clocks, void* stream) {
    const int64_t need = fmt == FMT_E4M3 ? 32 * 64 * 16 : 16 * 64 * 16;
    if (blocks <= 0 || iters <= 0 || ops == nullptr || sink == nullptr || ops_bytes < need ||
        reinterpret_cast<uintptr_t>(ops) % 16 != 0)
        return -1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4* o = static_cast<const u32x4*>(ops);
    switch (fmt) {
    case FMT_F16: hipLaunchKernelGGL(mfma_loop_kernel<FMT_F16>, dim3(blocks), dim3(256), 0, s, o, iters, sink, clocks); break;
    case FMT_BF16: hipLaunchKernelGGL(mfma_loop_kernel<FMT_BF16>, dim3(blocks), dim3(256), 0, s, o, iters, sink, clocks); break;
    case FMT_E4M3: hipLaunchKernelGGL(mfma_loop_kernel<FMT_E4M3>, dim3(blocks), dim3(256), 0, s, o, iters, sink, clocks); break;
    default: return -1;
    }
    return (int)hipGetLastError();
}

// FLOPs one call performs.
double bench_probe_flops(int fmt, int blocks, int iters) {
    return (double)blocks * 4 * iters * 32 * (fmt == FMT_E4M3 ? 131072.0 : 32768.0);
}

}  // extern "C"
