// Split-K GEMM into F32 partial slabs for gfx950 (CDNA4).
//
// partials[s,i,j] = sum over k in [s*kps, min((s+1)*kps, K)) of A[i,k]*B[j,k]
// ("Aligned shared rows for pipelined NAX on CUDA", section "Contract and
// correctness"; "Wider consecutive-weight NAX GEMM", section "Launch contract
// and correctness").  A is [M,K], B is [N,K], both k-contiguous.
//
// The pages' own kernels (a 32x64 tile on 128 threads, 40-element padded
// shared rows, BF16 converted to F16 on the way in) were built for other
// hardware.  What is kept here is the contract.  The design is:
//
//  * Native MFMA on the stored element type: v_mfma_f32_32x32x16_{bf16,f16}
//    for 16-bit inputs and v_mfma_f32_32x32x2_f32 for F32, accumulating in
//    F32.  BF16 is never narrowed to F16.
//  * Both operands are k-contiguous, so both MFMA fragments can be fetched
//    straight from global memory: lane l (row l%32 of a 32-row block, half
//    h = l/32) reads 64 consecutive bytes of its row per 128-byte chunk, as
//    four 16-byte loads.  Piece q of that read feeds MFMA step q.  The order
//    in which an MFMA's k slots are filled does not change the dot product,
//    so A and B fragments only have to use the same slot -> k assignment,
//    which they do because they are loaded identically.
//  * In the skinny shapes of this workload the grid has only a few hundred
//    output tiles, so the k axis of each split is shared among the waves of
//    a workgroup (chunk c goes to wave c % W) and the W partial tiles are
//    added through LDS in a fixed wave order before one coalesced 16-byte
//    store per lane.  No atomics; every output element is written once.
//  * Slice ends are multiples of 32 elements.  For 16-bit inputs a chunk is
//    64 elements, so the last chunk of a slice may be half empty: those lanes
//    skip their loads (exec-masked) and feed zeros, which adds exactly 0.
//    No load ever touches memory past the slice, so the exact-extent rule
//    holds for the last split of the last row.
//  * Workgroups are renumbered so that the tiles sharing a B panel (same
//    split and column block, different row blocks) land on one XCD and reuse
//    it from that XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitk_internal.h"

namespace splitk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunkBytes = 128;  // one chunk: 128 bytes of a row
constexpr int kHalfBytes = 64;    // the part of a chunk one lane reads
constexpr int kPieces = 4;        // 16-byte loads per lane per chunk and block

// Element-type specific MFMA step on one 16-byte piece of each operand.
template <int DT>
struct Mfma;

template <>
struct Mfma<2> {  // BF16: one 32x32x16 MFMA per 8-element piece
    static constexpr int kElemBytes = 2;
    static constexpr int kStepsPerPiece = 1;
    __device__ static inline f32x16 step(u32x4 a, u32x4 b, f32x16 c, int) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <>
struct Mfma<1> {  // F16: one 32x32x16 MFMA per 8-element piece
    static constexpr int kElemBytes = 2;
    static constexpr int kStepsPerPiece = 1;
    __device__ static inline f32x16 step(u32x4 a, u32x4 b, f32x16 c, int) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                       __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

template <>
struct Mfma<0> {  // F32: four 32x32x2 MFMAs per 4-element piece, one element each
    static constexpr int kElemBytes = 4;
    static constexpr int kStepsPerPiece = 4;
    __device__ static inline f32x16 step(u32x4 a, u32x4 b, f32x16 c, int e) {
        // Extract the element into a scalar before reinterpreting it: a bit
        // cast applied directly to a vector-element expression reads element 0.
        const uint32_t ua = a[e], ub = b[e];
        return __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(ua), __uint_as_float(ub), c, 0,
                                                     0, 0);
    }
};

// Renumbers workgroups so that consecutive logical ids run on one XCD.
// Workgroup b is dispatched to XCD b % 8; logical ids [start_x, start_x+cnt_x)
// go to XCD x.  It is a bijection on [0, n) whatever the dispatch order.
__device__ inline int xcd_logical_id(int b, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = b & 7, slot = b >> 3;
    return x < r ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
}

template <int DT, int BM, int BN, int W>
__global__ __launch_bounds__(W * 64) void gemm_bt_wavek(const uint8_t* __restrict__ A,
                                                        const uint8_t* __restrict__ B,
                                                        float* __restrict__ P, int M, int N, int K,
                                                        int kps, int tiles_m, int tiles_n) {
    using Op = Mfma<DT>;
    constexpr int ES = Op::kElemBytes;
    constexpr int CK = kChunkBytes / ES;  // elements per chunk
    constexpr int MB = BM / 32, NB = BN / 32;
    constexpr int PITCH = BN + 8;  // floats per row of the LDS reduction tile
    __shared__ float red[W][BM][PITCH];

    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    const int mt = logical % tiles_m;
    const int rest = logical / tiles_m;
    const int nt = rest % tiles_n;
    const int s = rest / tiles_n;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 31;
    const int h = lane >> 5;

    const int k0 = s * kps;
    const int k1 = min(k0 + kps, K);
    const int nchunks = (k1 - k0 + CK - 1) / CK;

    const size_t row_bytes = (size_t)K * ES;
    const uint8_t* a_row[MB];
    const uint8_t* b_row[NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        a_row[mb] = A + (size_t)(mt * BM + mb * 32 + r) * row_bytes + (size_t)k0 * ES + h * kHalfBytes;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        b_row[nb] = B + (size_t)(nt * BN + nb * 32 + r) * row_bytes + (size_t)k0 * ES + h * kHalfBytes;

    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};

    u32x4 av[MB][kPieces], bv[NB][kPieces];
    auto load = [&](int c) {
        // This lane's half of chunk c holds elements starting at k0 + c*CK + h*CK/2.
        const bool valid = c < nchunks && (k0 + c * CK + h * (CK / 2)) < k1;
        const size_t off = (size_t)c * kChunkBytes;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < kPieces; ++q)
                av[mb][q] = valid ? *(const u32x4*)(a_row[mb] + off + q * 16) : u32x4{};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < kPieces; ++q)
                bv[nb][q] = valid ? *(const u32x4*)(b_row[nb] + off + q * 16) : u32x4{};
    };

    if (wave < nchunks) load(wave);
    for (int c = wave; c < nchunks; c += W) {
        u32x4 ca[MB][kPieces], cb[NB][kPieces];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int q = 0; q < kPieces; ++q) ca[mb][q] = av[mb][q];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < kPieces; ++q) cb[nb][q] = bv[nb][q];
        if (c + W < nchunks) load(c + W);  // prefetch the next chunk of this wave
#pragma unroll
        for (int q = 0; q < kPieces; ++q)
#pragma unroll
            for (int e = 0; e < Op::kStepsPerPiece; ++e)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[mb][nb] = Op::step(ca[mb][q], cb[nb][q], acc[mb][nb], e);
    }

    // 32x32 accumulator layout: register i of lane l holds
    // row 8*(i/4) + 4*(l/32) + i%4, column l%32 of the block.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                red[wave][mb * 32 + 8 * (i >> 2) + 4 * h + (i & 3)][nb * 32 + r] = acc[mb][nb][i];
    __syncthreads();

    // Sum the W partial tiles in ascending wave order; one 16-byte store per item.
    constexpr int ROW4 = BN / 4;
    float* out = P + ((size_t)s * M + (size_t)mt * BM) * N + (size_t)nt * BN;
    for (int it = threadIdx.x; it < BM * ROW4; it += W * 64) {
        const int row = it / ROW4;
        const int col = (it % ROW4) * 4;
        f32x4 v = *(const f32x4*)&red[0][row][col];
#pragma unroll
        for (int w = 1; w < W; ++w) v += *(const f32x4*)&red[w][row][col];
        *(f32x4*)(out + (size_t)row * N + col) = v;
    }
}

template <int DT, int BM, int BN, int W>
hipError_t launch_wavek(const void* A, const void* B, float* P, int64_t M, int64_t N, int64_t K,
                        int64_t kps, int64_t splits, hipStream_t stream) {
    const int tiles_m = (int)(M / BM), tiles_n = (int)(N / BN);
    const dim3 grid((unsigned)(tiles_m * (int64_t)tiles_n * splits));
    const dim3 block(W * 64);
    const uint8_t* a = (const uint8_t*)A;
    const uint8_t* b = (const uint8_t*)B;
    int m = (int)M, n = (int)N, k = (int)K, kp = (int)kps;
    void* args[] = {&a, &b, &P, &m, &n, &k, &kp, (void*)&tiles_m, (void*)&tiles_n};
    return hipLaunchKernel((const void*)&gemm_bt_wavek<DT, BM, BN, W>, grid, block, args, 0, stream);
}

template <int DT>
hipError_t launch_dtype(const GemmPlan& p, const void* A, const void* B, float* P, int64_t M,
                        int64_t N, int64_t K, int64_t kps, int64_t splits, hipStream_t st) {
    if (p.kind == kWaveK && p.waves == 4) {
        if (p.bm == 32 && p.bn == 32) return launch_wavek<DT, 32, 32, 4>(A, B, P, M, N, K, kps, splits, st);
        if (p.bm == 32 && p.bn == 64) return launch_wavek<DT, 32, 64, 4>(A, B, P, M, N, K, kps, splits, st);
    }
    return hipErrorInvalidConfiguration;
}

}  // namespace

GemmPlan plan_gemm(int dtype, int64_t M, int64_t N, int64_t K, int64_t kps, int64_t splits) {
    (void)K;
    const int64_t es = dtype == 0 ? 4 : 2;
    // Pick the tile that moves the fewest bytes through the busiest CU: each
    // workgroup streams (BM + BN) rows of its split, and workgroups beyond the
    // 256 CUs queue behind the first round.
    struct Cand { int bm, bn; };
    const Cand cands[] = {{32, 64}, {32, 32}};
    GemmPlan best{kWaveK, 32, 32, 4, 0, 256};
    int64_t best_cost = -1;
    for (const Cand& c : cands) {
        if (M % c.bm || N % c.bn) continue;
        const int64_t wg = (M / c.bm) * (N / c.bn) * splits;
        const int64_t rounds = (wg + 255) / 256;
        const int64_t cost = rounds * (c.bm + c.bn) * kps * es;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = GemmPlan{kWaveK, c.bm, c.bn, 4, wg, 4 * 64};
        }
    }
    return best;
}

hipError_t launch_gemm_bt(const GemmPlan& plan, const void* A, const void* B, float* partials,
                          int64_t M, int64_t N, int64_t K, int64_t kps, int64_t splits, int dtype,
                          hipStream_t stream) {
    switch (dtype) {
        case 0: return launch_dtype<0>(plan, A, B, partials, M, N, K, kps, splits, stream);
        case 1: return launch_dtype<1>(plan, A, B, partials, M, N, K, kps, splits, stream);
        case 2: return launch_dtype<2>(plan, A, B, partials, M, N, K, kps, splits, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace splitk
