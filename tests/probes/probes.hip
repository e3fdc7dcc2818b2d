// probes.hip -- small gfx950 kernels that record how an instruction
// distributes data over the 64 lanes of a wave, so the tests can pin the
// lane layouts the GEMM kernels rely on (the unique-value ownership probe of
// "mma.sync and ldmatrix", section "Two probes and one matmul": fill the
// tiles with one distinct value per cell and let the host name the
// coordinate every lane received).
//
// Every probe runs one wave (64 lanes), keeps all accesses inside its own
// buffers (addresses are masked in-kernel as well as checked on the host),
// and synchronises before returning.  Test infrastructure only.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b8: LDS byte i holds (i >> shift) & 255 (two runs, shift 0
// and 8, name the source byte of every result byte).  Lane l reads at byte
// address addr[l] (8-byte aligned, < 2048); out[8l+j] receives byte j of the
// lane's 8-byte result.
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
__global__ void probe_tr8_kernel(const int32_t* addr, int shift, uint8_t* out) {
    __shared__ uint8_t lds[2048];
    const int l = threadIdx.x;
    for (int i = l; i < 2048; i += 64) lds[i] = (uint8_t)((i >> shift) & 255);
    __syncthreads();
    const int a = addr[l] & 2040;                 // in range and 8-byte aligned
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2*)((__attribute__((address_space(3))) uint8_t*)lds + a));
    for (int j = 0; j < 8; ++j) out[8 * l + j] = (uint8_t)((uint32_t)v[j >> 2] >> (8 * (j & 3)));
}

// ds_read_b64_tr_b16: LDS holds 1024 16-bit values equal to their index.
// Lane l reads at byte address addr[l] (8-byte aligned, < 2048); out[4l+j]
// receives element j of the lane's result.
__global__ void probe_tr16_kernel(const int32_t* addr, int16_t* out) {
    __shared__ short lds[1024];
    const int l = threadIdx.x;
    for (int i = l; i < 1024; i += 64) lds[i] = (short)i;
    __syncthreads();
    const int a = addr[l] & 2040;                 // in range and 8-byte aligned
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)lds + a));
    for (int j = 0; j < 4; ++j) out[4 * l + j] = v[j];
}

// global_load_lds_dwordx4: LDS (4096 bytes) is cleared, then every lane
// loads the 16 bytes src[4*src_chunk[l] .. +3] (src holds 64 chunks) into
// LDS through the instruction with LDS base `base` (bytes, 16-aligned,
// <= 3072).  out receives the whole LDS image (1024 dwords).
__global__ void probe_load_lds_kernel(const uint32_t* src, const int32_t* src_chunk, int base,
                                      uint32_t* out) {
    __shared__ uint32_t lds[1024];
    const int l = threadIdx.x;
    for (int i = l; i < 1024; i += 64) lds[i] = 0xFFFFFFFFu;
    __syncthreads();
    const int c = src_chunk[l] & 63;
    const int b = base & 3056;
    __builtin_amdgcn_global_load_lds(src + 4 * c, lds + b / 4, 16, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int i = l; i < 1024; i += 64) out[i] = lds[i];
}

// v_mfma_f32_32x32x16_{f16,bf16} and v_mfma_f32_16x16x32_{f16,bf16} with
// operands taken straight from lane registers: a[8l+j], b[8l+j] are lane l's
// operand elements (bit patterns); d receives the accumulator registers,
// d[16l+i] (32x32) or d[4l+i] (16x16).
template <bool BF16, bool BIG>
__global__ void probe_mfma_kernel(const uint16_t* a, const uint16_t* b, float* d) {
    const int l = threadIdx.x;
    u32x4 av, bv;
    for (int j = 0; j < 4; ++j) {
        av[j] = (uint32_t)a[8 * l + 2 * j] | ((uint32_t)a[8 * l + 2 * j + 1] << 16);
        bv[j] = (uint32_t)b[8 * l + 2 * j] | ((uint32_t)b[8 * l + 2 * j + 1] << 16);
    }
    if constexpr (BIG) {
        f32x16 acc = {};
        if constexpr (BF16)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
        else
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                         __builtin_bit_cast(f16x8, bv), acc, 0, 0, 0);
        for (int i = 0; i < 16; ++i) d[16 * l + i] = acc[i];
    } else {
        f32x4 acc = {};
        if constexpr (BF16)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
        else
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, av),
                                                         __builtin_bit_cast(f16x8, bv), acc, 0, 0, 0);
        for (int i = 0; i < 4; ++i) d[4 * l + i] = acc[i];
    }
}

// Back-to-back independent MFMAs on register-resident operands, timed with
// the shader clock (s_memtime) by lane 0 of every wave: cycles[w] for
// `iters` x 8 MFMAs of one wave.  Launch with any number of 256-lane blocks.
template <bool BF16>
__global__ __launch_bounds__(256) void probe_mfma_rate_kernel(int iters, uint64_t* cycles, float* sink) {
    u32x4 av = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
    u32x4 bv = av;
    f32x16 acc[8];
    for (int i = 0; i < 8; ++i) acc[i] = (f32x16){};
    __syncthreads();
    const uint64_t t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (BF16)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                                 __builtin_bit_cast(bf16x8, bv), acc[i], 0, 0, 0);
            else
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                                __builtin_bit_cast(f16x8, bv), acc[i], 0, 0, 0);
        }
    }
    float s = 0.0f;
    for (int i = 0; i < 8; ++i) s += acc[i][0];
    const uint64_t t1 = __builtin_readcyclecounter();
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if ((threadIdx.x & 63) == 0) cycles[wave] = t1 - t0;
    if (s == 12345.0f) sink[0] = s;
}

// The same MFMA stream fed with data: every lane loads 16 operand register
// sets (8 for A, 8 for B, 16 bytes each) from ops[16 * 64] and the MFMAs of
// one iteration rotate through them, so consecutive MFMAs see different
// operands as in a GEMM's k-loop (the constant-operand kernel above keeps the
// multiplier inputs still).  iters x 32 MFMAs per wave; one wave per SIMD.
template <bool BF16>
__global__ __launch_bounds__(256, 1) void probe_mfma_data_kernel(const u32x4* ops, int iters, float* sink) {
    const int l = threadIdx.x & 63;
    u32x4 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = ops[(2 * i) * 64 + l];
        b[i] = ops[(2 * i + 1) * 64 + l];
    }
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (f32x16){};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const u32x4 av = a[(i + r) & 7], bv = b[(i + 3 * r) & 7];
                if constexpr (BF16)
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av),
                                                                     __builtin_bit_cast(bf16x8, bv), acc[i], 0, 0, 0);
                else
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                                    __builtin_bit_cast(f16x8, bv), acc[i], 0, 0, 0);
            }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
    if (s == 12345.0f) sink[0] = s;
}

// v_mfma_f32_32x32x64_f8f6f4 with both operands in one 8-bit float format
// (FMT 0: E4M3, 1: E5M2; zero scale operands select the unscaled form).
// Lane l's 32 operand bytes are a[32l .. 32l+31] and b[32l .. 32l+31];
// d[16l + i] receives accumulator element i of lane l.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
template <int FMT>
__global__ void probe_mfma_f8_kernel(const uint32_t* a, const uint32_t* b, float* d) {
    const int l = threadIdx.x;
    i32x8 av, bv;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        av[j] = (int32_t)a[8 * l + j];
        bv[j] = (int32_t)b[8 * l + j];
    }
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, FMT, FMT, 0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) d[16 * l + i] = acc[i];
}

// The same MFMA with an incoming accumulator: d = c + A.B, with c[16l + i]
// the accumulator element i of lane l (the 32x32 accumulator map).
template <int FMT>
__global__ void probe_mfma_f8_acc_kernel(const uint32_t* a, const uint32_t* b, const float* c, float* d) {
    const int l = threadIdx.x;
    i32x8 av, bv;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        av[j] = (int32_t)a[8 * l + j];
        bv[j] = (int32_t)b[8 * l + j];
    }
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = c[16 * l + i];
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, FMT, FMT, 0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) d[16 * l + i] = acc[i];
}

// Issue rate of v_mfma_f32_32x32x64_f8f6f4 (E4M3), as probe_mfma_rate_kernel:
// eight independent accumulators, register-resident operands.
__global__ __launch_bounds__(256) void probe_mfma_f8_rate_kernel(int iters, uint64_t* cycles, float* sink) {
    i32x8 av = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838};
    i32x8 bv = av;
    f32x16 acc[8];
    for (int i = 0; i < 8; ++i) acc[i] = (f32x16){};
    __syncthreads();
    const uint64_t t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i], 0, 0, 0, 0, 0, 0);
    }
    float s = 0.0f;
    for (int i = 0; i < 8; ++i) s += acc[i][0];
    const uint64_t t1 = __builtin_readcyclecounter();
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    if ((threadIdx.x & 63) == 0) cycles[wave] = t1 - t0;
    if (s == 12345.0f) sink[0] = s;
}

// The 8-bit form of the data-fed stream: v_mfma_f32_32x32x64_f8f6f4 (E4M3),
// 8 operand register sets of 32 bytes per lane for A and for B from
// ops[16 * 2 * 64] (16-byte units), rotating as above; iters x 32 MFMAs per wave.
__global__ __launch_bounds__(256, 1) void probe_mfma_data_f8_kernel(const u32x4* ops, int iters, float* sink) {
    const int l = threadIdx.x & 63;
    i32x8 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u32x4 a0 = ops[(4 * i) * 64 + l], a1 = ops[(4 * i + 1) * 64 + l];
        const u32x4 b0 = ops[(4 * i + 2) * 64 + l], b1 = ops[(4 * i + 3) * 64 + l];
        a[i] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        b[i] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    }
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (f32x16){};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(i + r) & 7], b[(i + 3 * r) & 7], acc[i],
                                                                         0, 0, 0, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
    if (s == 12345.0f) sink[0] = s;
}

// LDS throughput: every wave of 4 per block issues `iters` x 8 LDS
// instructions of one kind and lane 0 records the shader cycles.  Lane l of
// wave w uses byte address addr[64 w + l] (masked to the 64 KiB buffer and
// to the access size), moved by (it & 3) << 14 each iteration so nothing can
// be hoisted, and by u * 8192 for the 8 unrolled instructions.
//   kind 0: ds_read_b128   1: ds_read_b64   2: ds_read_b64_tr_b16
//   kind 3: ds_write_b128
template <int KIND>
__global__ __launch_bounds__(256) void probe_lds_rate_kernel(int iters, const int32_t* addr_table,
                                                             uint64_t* cycles, uint32_t* sink) {
    __shared__ __attribute__((aligned(1024))) char lds[65536];
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 65536 / 4; i += 256) reinterpret_cast<uint32_t*>(lds)[i] = i;
    const int align = (KIND == 0 || KIND == 3) ? 16 : 8;
    const int addr = addr_table[threadIdx.x] & 65535 & ~(align - 1);
    uint32_t x = 0;
    u32x4 wv = {(uint32_t)l, 1u, 2u, 3u};
    __syncthreads();
    const uint64_t t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
        const int base = addr + ((it & 3) << 14);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int a = (base + u * 8192) & 65535;
            if constexpr (KIND == 0) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(lds + a);
                x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
            } else if constexpr (KIND == 1) {
                const uint64_t v = *reinterpret_cast<const uint64_t*>(lds + a);
                x ^= (uint32_t)v ^ (uint32_t)(v >> 32);
            } else if constexpr (KIND == 3) {
                wv[1] ^= (uint32_t)it;
                *reinterpret_cast<u32x4*>(lds + a) = wv;
            } else {
                const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)lds + a));
                const u32x2 v2 = __builtin_bit_cast(u32x2, v);
                x ^= v2[0] ^ v2[1];
            }
        }
    }
    const uint64_t t1 = __builtin_readcyclecounter();
    if (l == 0) cycles[blockIdx.x * 4 + w] = t1 - t0;
    if (KIND == 3) x = reinterpret_cast<const uint32_t*>(lds)[threadIdx.x];
    if (x == 0x12345678u) sink[0] = x;
}

// Global -> LDS copy throughput: every wave of 4 per block issues `iters` x 8
// global_load_lds_dwordx4 (1 KiB each) from a source of `src_bytes` bytes
// (a power of two, at least 8 KiB; small enough to stay in L2) into its own
// 8 KiB of LDS, waits for all of them, and lane 0 records the shader cycles.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__global__ __launch_bounds__(256) void probe_dma_rate_kernel(int iters, const char* src, int src_bytes,
                                                             uint64_t* cycles, uint32_t* sink) {
    __shared__ __attribute__((aligned(1024))) char lds[32768];
    const int l = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t base = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)lds + w * 8192;
    const int mask = src_bytes - 1;
    __syncthreads();
    const uint64_t t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const char* p = src + (((it * 8 + u) * 1024 + w * 65536 + blockIdx.x * 4096 + l * 16) & mask);
            asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                         :: "v"(p), "s"(base + u * 1024) : "memory", "m0");
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint64_t t1 = __builtin_readcyclecounter();
    if (l == 0) cycles[blockIdx.x * 4 + w] = t1 - t0;
    __syncthreads();
    if (reinterpret_cast<const uint32_t*>(lds)[threadIdx.x] == 0x12345678u) sink[0] = 1;
}
#pragma clang diagnostic pop

// LDS read throughput against parallelism: blockDim.x / 64 waves per CU, each
// issuing `iters` x UNROLL independent reads.  KIND 0: ds_read_b128 on
// consecutive 16-byte chunks; 1: ds_read_b64_tr_b16 with the GEMM's
// B-fragment addressing (rows of 512 bytes, chunk ^ 2(k&3)).  Addresses stay
// inside the 64 KiB buffer.
template <int KIND, int UNROLL>
__global__ __launch_bounds__(1024) void probe_lds_par_kernel(int iters, uint64_t* cycles, uint32_t* sink) {
    __shared__ __attribute__((aligned(1024))) char lds[65536];
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < 65536 / 4; i += blockDim.x) reinterpret_cast<uint32_t*>(lds)[i] = i;
    int addr;
    if (KIND == 0) {
        addr = (w * 1024 + l * 16) & 65535;
    } else {
        const int g = l >> 4, ip = l & 15;
        const int k = 8 * (g >> 1) + (ip >> 2) + 16 * ((w >> 1) & 3);
        const int n = 16 * (g & 1) + 4 * (ip & 3) + 128 * (w & 1);
        addr = k * 512 + (((n >> 3) ^ (2 * (k & 3))) * 16) + (n & 7) * 2;
    }
    uint32_t x = 0;
    __syncthreads();
    const uint64_t t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
        const int base = addr + ((it & 1) << 15);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int a = (base + u * 2048) & 65535;
            if constexpr (KIND == 0) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (a & ~15));
                x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
            } else {
                const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) char*)lds + (a & ~7)));
                const u32x2 v2 = __builtin_bit_cast(u32x2, v);
                x ^= v2[0] ^ v2[1];
            }
        }
    }
    const uint64_t t1 = __builtin_readcyclecounter();
    if (l == 0) cycles[blockIdx.x * 16 + w] = t1 - t0;
    if (x == 0x12345678u) sink[0] = x;
}

// 16-byte global loads from addresses that are only 2-byte aligned: lane l
// reads the 16 bytes at src + offset + 32 l with global_load_dwordx4 (into
// out_vec[4l..4l+3]) and with global_load_lds_dwordx4 (LDS image copied to
// out_lds[4l..4l+3]).  src must hold at least offset + 32*64 + 16 bytes; the
// host checks it.  Either the bytes at the exact address come back, or (in
// strict alignment mode) those of the aligned-down address: no fault either way.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__global__ void probe_unaligned_kernel(const char* src, int offset, uint32_t* out_vec, uint32_t* out_lds) {
    __shared__ __attribute__((aligned(1024))) uint32_t lds[256];
    const int l = threadIdx.x;
    const char* p = src + offset + 32 * l;
    u32x4 v;
    asm volatile("global_load_dwordx4 %0, %1, off\n\ts_waitcnt vmcnt(0)" : "=v"(v) : "v"(p) : "memory");
    for (int j = 0; j < 4; ++j) out_vec[4 * l + j] = v[j];
    lds[l] = 0; lds[64 + l] = 0; lds[128 + l] = 0; lds[192 + l] = 0;
    __syncthreads();
    const uint32_t base = (uint32_t)(size_t)(__attribute__((address_space(3))) uint32_t*)lds;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off\n\ts_waitcnt vmcnt(0)"
                 :: "v"(p), "s"(base) : "memory", "m0");
    __syncthreads();
    for (int j = 0; j < 4; ++j) out_lds[4 * l + j] = lds[4 * l + j];
}
// The lane exchange of the whole-tile epilogues: v_permlane32_swap_b32 in
// the kernels' form (s_nop 1 before and after) on x = 1000 + lane and
// y = 2000 + lane; out[0..63] = x afterwards, out[64..127] = y afterwards.
__global__ void probe_permlane32_swap_kernel(uint32_t* out) {
    const uint32_t l = threadIdx.x;
    uint32_t x = 1000u + l, y = 2000u + l;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
    out[l] = x;
    out[64 + l] = y;
}
#pragma clang diagnostic pop

extern "C" {

int probe_permlane32_swap(uint32_t* out) {
    hipLaunchKernelGGL(probe_permlane32_swap_kernel, dim3(1), dim3(64), 0, 0, out);
    return (int)hipDeviceSynchronize();
}

int probe_unaligned(const char* src, int src_bytes, int offset, uint32_t* out_vec, uint32_t* out_lds) {
    if (offset < 0 || offset + 32 * 64 + 16 > src_bytes) return -1;
    hipLaunchKernelGGL(probe_unaligned_kernel, dim3(1), dim3(64), 0, 0, src, offset, out_vec, out_lds);
    return (int)hipDeviceSynchronize();
}

// cycles must hold blocks * 16 entries; threads in {256, 512, 1024}.
int probe_lds_par(int kind, int unroll16, int blocks, int threads, int iters, uint64_t* cycles, uint32_t* sink) {
    if (threads != 256 && threads != 512 && threads != 1024) return -1;
    const dim3 g(blocks), b(threads);
    if (kind == 0 && !unroll16) hipLaunchKernelGGL((probe_lds_par_kernel<0, 8>), g, b, 0, 0, iters, cycles, sink);
    else if (kind == 0) hipLaunchKernelGGL((probe_lds_par_kernel<0, 16>), g, b, 0, 0, iters, cycles, sink);
    else if (!unroll16) hipLaunchKernelGGL((probe_lds_par_kernel<1, 8>), g, b, 0, 0, iters, cycles, sink);
    else hipLaunchKernelGGL((probe_lds_par_kernel<1, 16>), g, b, 0, 0, iters, cycles, sink);
    return (int)hipDeviceSynchronize();
}

int probe_dma_rate(int blocks, int iters, const char* src, int src_bytes, uint64_t* cycles, uint32_t* sink) {
    if (src_bytes < 8192 || (src_bytes & (src_bytes - 1)) != 0) return -1;
    hipLaunchKernelGGL(probe_dma_rate_kernel, dim3(blocks), dim3(256), 0, 0, iters, src, src_bytes, cycles, sink);
    return (int)hipDeviceSynchronize();
}

int probe_lds_rate(int kind, int blocks, int iters, const int32_t* addr_table, uint64_t* cycles,
                   uint32_t* sink) {
    switch (kind) {
    case 0: hipLaunchKernelGGL(probe_lds_rate_kernel<0>, dim3(blocks), dim3(256), 0, 0, iters, addr_table, cycles, sink); break;
    case 1: hipLaunchKernelGGL(probe_lds_rate_kernel<1>, dim3(blocks), dim3(256), 0, 0, iters, addr_table, cycles, sink); break;
    case 2: hipLaunchKernelGGL(probe_lds_rate_kernel<2>, dim3(blocks), dim3(256), 0, 0, iters, addr_table, cycles, sink); break;
    default: hipLaunchKernelGGL(probe_lds_rate_kernel<3>, dim3(blocks), dim3(256), 0, 0, iters, addr_table, cycles, sink); break;
    }
    return (int)hipDeviceSynchronize();
}

int probe_tr16(const int32_t* addr, int16_t* out) {
    hipLaunchKernelGGL(probe_tr16_kernel, dim3(1), dim3(64), 0, 0, addr, out);
    return (int)hipDeviceSynchronize();
}

int probe_tr8(const int32_t* addr, int shift, uint8_t* out) {
    hipLaunchKernelGGL(probe_tr8_kernel, dim3(1), dim3(64), 0, 0, addr, shift, out);
    return (int)hipDeviceSynchronize();
}

int probe_load_lds(const uint32_t* src, const int32_t* src_chunk, int base, uint32_t* out) {
    hipLaunchKernelGGL(probe_load_lds_kernel, dim3(1), dim3(64), 0, 0, src, src_chunk, base, out);
    return (int)hipDeviceSynchronize();
}

// kind: 0 f16 32x32x16, 1 bf16 32x32x16, 2 f16 16x16x32, 3 bf16 16x16x32
int probe_mfma(int kind, const uint16_t* a, const uint16_t* b, float* d) {
    switch (kind) {
    case 0: hipLaunchKernelGGL((probe_mfma_kernel<false, true>), dim3(1), dim3(64), 0, 0, a, b, d); break;
    case 1: hipLaunchKernelGGL((probe_mfma_kernel<true, true>), dim3(1), dim3(64), 0, 0, a, b, d); break;
    case 2: hipLaunchKernelGGL((probe_mfma_kernel<false, false>), dim3(1), dim3(64), 0, 0, a, b, d); break;
    default: hipLaunchKernelGGL((probe_mfma_kernel<true, false>), dim3(1), dim3(64), 0, 0, a, b, d); break;
    }
    return (int)hipDeviceSynchronize();
}

int probe_mfma_rate(int bf16, int blocks, int iters, uint64_t* cycles, float* sink) {
    if (bf16)
        hipLaunchKernelGGL(probe_mfma_rate_kernel<true>, dim3(blocks), dim3(256), 0, 0, iters, cycles, sink);
    else
        hipLaunchKernelGGL(probe_mfma_rate_kernel<false>, dim3(blocks), dim3(256), 0, 0, iters, cycles, sink);
    return (int)hipDeviceSynchronize();
}

// ops: 16 x 64 lanes x 16 bytes of fp16 (bf16 = 0) or bf16 (bf16 = 1) values.
int probe_mfma_data(int bf16, int blocks, int iters, const void* ops, float* sink) {
    const u32x4* o = (const u32x4*)ops;
    if (bf16)
        hipLaunchKernelGGL(probe_mfma_data_kernel<true>, dim3(blocks), dim3(256), 0, 0, o, iters, sink);
    else
        hipLaunchKernelGGL(probe_mfma_data_kernel<false>, dim3(blocks), dim3(256), 0, 0, o, iters, sink);
    return (int)hipDeviceSynchronize();
}

// fmt: 0 E4M3, 1 E5M2.  a, b: 64 lanes x 32 bytes; d: 64 x 16 floats.
int probe_mfma_f8(int fmt, const uint32_t* a, const uint32_t* b, float* d) {
    if (fmt == 0)
        hipLaunchKernelGGL(probe_mfma_f8_kernel<0>, dim3(1), dim3(64), 0, 0, a, b, d);
    else
        hipLaunchKernelGGL(probe_mfma_f8_kernel<1>, dim3(1), dim3(64), 0, 0, a, b, d);
    return (int)hipDeviceSynchronize();
}

int probe_mfma_f8_acc(int fmt, const uint32_t* a, const uint32_t* b, const float* c, float* d) {
    if (fmt == 0)
        hipLaunchKernelGGL(probe_mfma_f8_acc_kernel<0>, dim3(1), dim3(64), 0, 0, a, b, c, d);
    else
        hipLaunchKernelGGL(probe_mfma_f8_acc_kernel<1>, dim3(1), dim3(64), 0, 0, a, b, c, d);
    return (int)hipDeviceSynchronize();
}

// ops: 32 x 64 lanes x 16 bytes of E4M3 values.
int probe_mfma_data_f8(int blocks, int iters, const void* ops, float* sink) {
    hipLaunchKernelGGL(probe_mfma_data_f8_kernel, dim3(blocks), dim3(256), 0, 0, (const u32x4*)ops, iters, sink);
    return (int)hipDeviceSynchronize();
}

int probe_mfma_f8_rate(int blocks, int iters, uint64_t* cycles, float* sink) {
    hipLaunchKernelGGL(probe_mfma_f8_rate_kernel, dim3(blocks), dim3(256), 0, 0, iters, cycles, sink);
    return (int)hipDeviceSynchronize();
}

}  // extern "C"
