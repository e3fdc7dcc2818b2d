// gemm_sk.hip -- split-K across workgroups: the work-splitting half of the
// stream-K idea of "The Asynchronous Kernel: Tensor Cores & TMA" (section
// "Keeping the line busy"), for outputs with too few 256x256 tiles to occupy
// the 256 CUs when K is long.
//
// The K range is cut into S pieces of Kc = ceil(K / S) rounded up to the
// slice depth (64 for 16-bit inputs, 128 for 8-bit ones; the last piece
// shorter), and the launch runs one workgroup per (tile, piece): each
// computes its tile's product over its piece of K with the 256x256
// direct-to-LDS tile of gemm_dl_kernel.h (dl_tile, unchanged: the piece is a
// smaller GEMM with the same leading dimensions, A offset by k0 columns and B
// by k0 rows, or k0 columns when B is column-major) and stores the fp32
// partial tile, 256 x 256 floats, into the caller's workspace.  A second
// kernel on the same stream sums the pieces of every output element in piece
// order (so the result does not depend on which workgroup finished first),
// applies the epilogue of the general form and rounds once to the output
// type.  Stream order is the only synchronisation: no atomics, no waits.
//
// Workspace layout: partial (s, tm, tn) at float offset
// ((s * tilesM + tm) * tilesN + tn) * 65536, row r of the tile at r * 256.
// Elements outside M x N are not written by the first kernel and are read,
// but never stored, by the second.
#include "gemm_dl_kernel.h"

namespace dhpt {
namespace sk {

using namespace dl;

constexpr int kTile = 256;
constexpr int64_t kTileFloats = (int64_t)kTile * kTile;

// Workgroup w: piece s = w / T, tile w % T in the grouped, XCD-aware order of
// a one-workgroup-per-tile launch (each piece's workgroups walk the tiles the
// way that launch does).
template <int IN, int EDGE, bool BT>
__global__ __launch_bounds__(256, 1) void gemm_sk_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    float* __restrict__ ws, int M, int N, int K, int Kc, int tilesM, int tilesN, int group_m) {
    constexpr int ESZ = kIn8<IN> ? 1 : 2;                // bytes per input element
    constexpr int FD = kIn8<IN> ? 1 : 2;                 // the 256x256 instance's fragment prefetch
    __shared__ __attribute__((aligned(1024))) char smem[dl_lds_bytes<IN, kTile, kTile, EDGE, BT>()];
    const int T = tilesM * tilesN;
    const int s = blockIdx.x / T;
    int tm, tn;
    tile_coords(blockIdx.x - s * T, tilesM, tilesN, group_m, &tm, &tn);
    const int m0 = tm * kTile, n0 = tn * kTile;
    const int k0 = s * Kc;
    const int Mt = M - m0 < kTile ? M - m0 : kTile;
    const int Nt = N - n0 < kTile ? N - n0 : kTile;
    const int Kt = K - k0 < Kc ? K - k0 : Kc;           // >= 1: the host launches only pieces inside K
    // element offsets, applied in bytes (the operands are byte streams of ESZ-byte elements)
    const char* Ab = reinterpret_cast<const char*>(A);
    const char* Bb = reinterpret_cast<const char*>(B);
    const uint16_t* As = reinterpret_cast<const uint16_t*>(Ab + ((int64_t)m0 * lda + k0) * ESZ);
    const uint16_t* Bs = reinterpret_cast<const uint16_t*>(
        Bb + (BT ? (int64_t)n0 * ldb + k0 : (int64_t)k0 * ldb + n0) * ESZ);
    float* P = ws + (((int64_t)s * tilesM + tm) * tilesN + tn) * kTileFloats;
    EpiArgs ep{1.0f, 0.0f, nullptr, 0};
#ifdef DHPT_TIMELINE
    ep.timeline = nullptr;
#endif
    dl_tile<IN, OUT_F32, kTile, kTile, FD, EDGE, BT, false, false>(smem, As, lda, Bs, ldb, P, kTile, Mt, Nt, Kt, 0,
                                                                  0, ep, (int)threadIdx.x);
}

// One thread per 4 consecutive columns of a row: the S partials of those 4
// elements (one 16-byte load each, partial rows are 256 floats), summed in
// piece order, the epilogue, one rounding, up to 4 stores.
template <int OUT, bool EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const float* __restrict__ ws, int S, void* __restrict__ C, int64_t ldc, int M, int N, int tilesM,
    int tilesN, EpiArgs ep) {
    const int n4 = (N + 3) / 4;
    const int64_t total = (int64_t)M * n4;
    const bool read_old = EPI && ep.beta != 0.0f;
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < total;
         it += (int64_t)gridDim.x * blockDim.x) {
        const int i = (int)(it / n4);
        const int j = (int)(it - (int64_t)i * n4) * 4;
        const int tm = i / kTile, tn = j / kTile;
        const int64_t in_tile = (int64_t)(i - tm * kTile) * kTile + (j - tn * kTile);
        const float4* p = reinterpret_cast<const float4*>(ws + ((int64_t)tm * tilesN + tn) * kTileFloats + in_tile);
        const int64_t piece = (int64_t)tilesM * tilesN * kTileFloats / 4;     // float4 stride between pieces
        // four pieces' loads in flight at a time, added strictly in piece order
        float4 acc = p[0];
        int s = 1;
        for (; s + 4 <= S; s += 4) {
            const float4 q0 = p[s * piece], q1 = p[(s + 1) * piece], q2 = p[(s + 2) * piece], q3 = p[(s + 3) * piece];
            acc.x += q0.x; acc.y += q0.y; acc.z += q0.z; acc.w += q0.w;
            acc.x += q1.x; acc.y += q1.y; acc.z += q1.z; acc.w += q1.w;
            acc.x += q2.x; acc.y += q2.y; acc.z += q2.z; acc.w += q2.w;
            acc.x += q3.x; acc.y += q3.y; acc.z += q3.z; acc.w += q3.w;
        }
        for (; s < S; ++s) {
            const float4 q = p[s * piece];
            acc.x += q.x; acc.y += q.y; acc.z += q.z; acc.w += q.w;
        }
        const float v[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = j + e;
            if (col < N) {
                const int64_t idx = (int64_t)i * ldc + col;
                float y = v[e];
                if constexpr (EPI) {
                    const float old = read_old ? load_out<OUT>(C, idx) : 0.0f;
                    y = epi_value(y, ep, read_old, old, ep.bias != nullptr ? ep.bias[col] : 0.0f);
                }
                store_out<OUT>(C, idx, y);
            }
        }
    }
}

template <int IN, int EDGE, bool BT>
static void launch_partial(const Problem& p, int pieces, int Kc, float* ws, int group_m, hipStream_t s) {
    const int tilesM = (p.M + kTile - 1) / kTile, tilesN = (p.N + kTile - 1) / kTile;
    hipLaunchKernelGGL((gemm_sk_kernel<IN, EDGE, BT>), dim3((unsigned)(tilesM * tilesN * pieces)), dim3(256),
                       0, s, p.A, p.lda, p.B, p.ldb, ws, p.M, p.N, p.K, Kc, tilesM, tilesN, group_m);
}

template <int OUT, bool EPI>
static void launch_reduce(const Problem& p, int pieces, const float* ws, hipStream_t s) {
    const int tilesM = (p.M + kTile - 1) / kTile, tilesN = (p.N + kTile - 1) / kTile;
    const int64_t items = (int64_t)p.M * ((p.N + 3) / 4);
    int64_t blocks = (items + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    EpiArgs ep{p.alpha, p.beta, p.bias, p.relu};
#ifdef DHPT_TIMELINE
    ep.timeline = nullptr;
#endif
    hipLaunchKernelGGL((splitk_reduce_kernel<OUT, EPI>), dim3((unsigned)blocks), dim3(256), 0, s, ws, pieces, p.C,
                       p.ldc, p.M, p.N, tilesM, tilesN, ep);
}

}  // namespace sk

// Pieces actually launched for `splits` requested: ceil(K / Kc), Kc a
// multiple of the slice depth `gran` (64 for 16-bit inputs, 128 for 8-bit).
int splitk_pieces(int K, int splits, int gran, int* Kc_out) {
    int64_t per = ((int64_t)K + splits - 1) / splits;
    const int Kc = (int)(((per + gran - 1) / gran) * gran);
    *Kc_out = Kc;
    return (int)(((int64_t)K + Kc - 1) / Kc);
}

hipError_t launch_splitk(const Problem& p, int splits, int edge, float* ws, int group_m, hipStream_t s) {
    using dl::IN_F16;
    using dl::IN_BF16;
    using dl::OUT_F32;
    using dl::OUT_F16;
    using dl::OUT_BF16;
    const bool in8 = dtype_in8(p.dtype);
    int Kc = 0;
    const int pieces = splitk_pieces(p.K, splits, in8 ? 128 : 64, &Kc);
    // input kind of each dtype (gemm_dtype_t order: f16, f16, bf16, bf16, then E4M3 x 3, E5M2 x 3)
    const int in = p.dtype <= 1 ? 0 : p.dtype <= 3 ? 1 : p.dtype <= 6 ? 2 : 3;
    auto by_input = [&](auto edge_c, auto bt_c) {
        constexpr int E = decltype(edge_c)::value;
        constexpr bool BT = decltype(bt_c)::value;
        switch (in) {
        case 0: sk::launch_partial<IN_F16, E, BT>(p, pieces, Kc, ws, group_m, s); break;
        case 1: sk::launch_partial<IN_BF16, E, BT>(p, pieces, Kc, ws, group_m, s); break;
        case 2: sk::launch_partial<dl::IN_E4M3, E, BT>(p, pieces, Kc, ws, group_m, s); break;
        default: sk::launch_partial<dl::IN_E5M2, E, BT>(p, pieces, Kc, ws, group_m, s); break;
        }
    };
    auto partial = [&](auto edge_c) {
        if (p.transB) by_input(edge_c, std::true_type{});
        else by_input(edge_c, std::false_type{});
    };
    if (edge == dl::EDGE_NONE) partial(std::integral_constant<int, dl::EDGE_NONE>{});
    else partial(std::integral_constant<int, dl::EDGE_CLAMP>{});
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // output kind of each dtype: f32, f16, f32, bf16, then (f32, f16, bf16) twice
    const int out = dtype_out_f32(p.dtype) ? OUT_F32 : (p.dtype == 1 || p.dtype == 5 || p.dtype == 8) ? OUT_F16
                                                                                                        : OUT_BF16;
    if (p.epi) {
        if (out == OUT_F32) sk::launch_reduce<OUT_F32, true>(p, pieces, ws, s);
        else if (out == OUT_F16) sk::launch_reduce<OUT_F16, true>(p, pieces, ws, s);
        else sk::launch_reduce<OUT_BF16, true>(p, pieces, ws, s);
    } else {
        if (out == OUT_F32) sk::launch_reduce<OUT_F32, false>(p, pieces, ws, s);
        else if (out == OUT_F16) sk::launch_reduce<OUT_F16, false>(p, pieces, ws, s);
        else sk::launch_reduce<OUT_BF16, false>(p, pieces, ws, s);
    }
    return hipGetLastError();
}

}  // namespace dhpt
