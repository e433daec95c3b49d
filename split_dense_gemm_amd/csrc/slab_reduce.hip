// Slab reduction: C[i,j] = sum over s of partials[s,i,j], in F32, stored as
// F32 or -- the typed final output -- rounded to F16 or BF16 (nearest, ties
// to even, by the hardware conversion instructions).
//
// This is the separate accumulation pass that follows the split-K GEMM
// ("Aligned shared rows for pipelined NAX on CUDA", sections "Contract and
// correctness" and "Measurement protocol"; "Wider consecutive-weight NAX
// GEMM", section "Performance method").  The pages do not describe it beyond
// being elementwise; here the slabs are added in ascending s with plain F32
// additions, so the result is deterministic.
//
// It reads splits*M*N*4 bytes and writes M*N*4 bytes once each, so it is
// bound by memory bandwidth.  A lane owns ITEMS 16-byte words of the [M*N]
// plane, spaced one grid apart, and issues every slab load of all of them
// before the first add, so ITEMS*S loads per lane are in flight together.
// Consecutive lanes touch consecutive words: every load and store
// instruction of a wave covers 1 KiB of contiguous memory.  The split count
// is a compile-time constant for 1..8 so that no load sits behind a branch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitk_internal.h"

namespace splitk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;

// Store of one 16-byte F32 word as output type OT (0 F32, 1 F16, 2 BF16),
// as a streaming (nontemporal) store when NT.
template <int OT, bool NT = false>
__device__ inline void store4(void* C, int64_t g, f32x4 v) {
    if constexpr (OT == 0) {
        if constexpr (NT) __builtin_nontemporal_store(v, &((f32x4*)C)[g]);
        else ((f32x4*)C)[g] = v;
    } else if constexpr (OT == 1) {
        const f16x4 h = __builtin_convertvector(v, f16x4);
        if constexpr (NT) __builtin_nontemporal_store(h, &((f16x4*)C)[g]);
        else ((f16x4*)C)[g] = h;
    } else {
        const bf16x4 h = __builtin_convertvector(v, bf16x4);
        if constexpr (NT) __builtin_nontemporal_store(h, &((bf16x4*)C)[g]);
        else ((bf16x4*)C)[g] = h;
    }
}

// Slab word load of the flat pass: streaming (nontemporal) when the slabs
// are too large for the memory-side cache (NT, see stream_slabs), normal
// otherwise.  Each word is read once.  With NT the sums are stored as
// streaming writes too: 8 slabs of 2048x4096 took 53.8 us with normal C
// stores and 50.7 us with streaming ones (a read-only pass over the same
// slabs takes 43.7 us).
template <bool NT>
__device__ inline f32x4 load_slab(const f32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <int S, int ITEMS, int OT, bool NT>
__global__ __launch_bounds__(kBlock) void slab_reduce_kernel(const f32x4* __restrict__ P,
                                                             void* __restrict__ C, int splits,
                                                             int64_t plane4) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    const int64_t g0 = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (S > 0) {
        f32x4 v[ITEMS][S > 0 ? S : 1];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t g = g0 + it * stride;
            if (g < plane4) {
#pragma unroll
                for (int s = 0; s < S; ++s) v[it][s] = load_slab<NT>(&P[s * plane4 + g]);
            }
        }
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t g = g0 + it * stride;
            if (g < plane4) {
                f32x4 acc = v[it][0];
#pragma unroll
                for (int s = 1; s < S; ++s) acc += v[it][s];
                store4<OT, NT>(C, g, acc);
            }
        }
    } else {
        // Any other split count: slabs in batches of eight whose loads are
        // all issued before their adds, still summed in ascending s.
        constexpr int kBatch = 8;
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t g = g0 + it * stride;
            if (g >= plane4) break;
            f32x4 acc = load_slab<NT>(&P[g]);
            int s = 1;
            for (; s + kBatch <= splits; s += kBatch) {
                f32x4 v[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) v[j] = load_slab<NT>(&P[(int64_t)(s + j) * plane4 + g]);
#pragma unroll
                for (int j = 0; j < kBatch; ++j) acc += v[j];
            }
            for (; s < splits; ++s) acc += load_slab<NT>(&P[(int64_t)s * plane4 + g]);
            store4<OT, NT>(C, g, acc);
        }
    }
}

template <int S, int ITEMS, int OT>
hipError_t launch(const float* partials, void* C, int splits, int64_t plane4, hipStream_t stream) {
    const int64_t per_block = (int64_t)kBlock * ITEMS;
    const dim3 grid((unsigned)((plane4 + per_block - 1) / per_block));
    const f32x4* p = (const f32x4*)partials;
    void* c = C;
    void* args[] = {&p, &c, &splits, &plane4};
    const bool nt = stream_slabs(splits, 1, plane4 * 4);
    return hipLaunchKernel(nt ? (const void*)&slab_reduce_kernel<S, ITEMS, OT, true>
                              : (const void*)&slab_reduce_kernel<S, ITEMS, OT, false>,
                           grid, dim3(kBlock), args, 0, stream);
}

template <int ITEMS, int OT>
hipError_t launch_items(const float* partials, void* C, int s, int64_t plane4, hipStream_t st) {
    switch (s) {
        case 1: return launch<1, ITEMS, OT>(partials, C, s, plane4, st);
        case 2: return launch<2, ITEMS, OT>(partials, C, s, plane4, st);
        case 3: return launch<3, ITEMS, OT>(partials, C, s, plane4, st);
        case 4: return launch<4, ITEMS, OT>(partials, C, s, plane4, st);
        case 5: return launch<5, ITEMS, OT>(partials, C, s, plane4, st);
        case 6: return launch<6, ITEMS, OT>(partials, C, s, plane4, st);
        case 7: return launch<7, ITEMS, OT>(partials, C, s, plane4, st);
        case 8: return launch<8, ITEMS, OT>(partials, C, s, plane4, st);
        default: return launch<0, ITEMS, OT>(partials, C, s, plane4, st);
    }
}

template <int OT>
hipError_t launch_out(const float* partials, void* C, int s, int64_t plane4, hipStream_t st) {
    // Four words per lane once the plane gives every CU several workgroups
    // that way (measured faster for large planes); one word per lane
    // otherwise, so that small planes still spread over all CUs.
    if (plane4 >= (int64_t)256 * 4 * kBlock * 4) return launch_items<4, OT>(partials, C, s, plane4, st);
    return launch_items<1, OT>(partials, C, s, plane4, st);
}

// Row bands per tile in the tile-ordered pass: one 16-byte word per lane.
constexpr int tile_bands(int bm, int bn) { return bm * bn / (4 * kBlock) > 1 ? bm * bn / (4 * kBlock) : 1; }

// Tile-ordered pass for the slabs of a GEMM in the split-fastest order (BM x
// BN output tiles, tiles_m of them down M: the skinny tiles, and 256x128 or
// 256x256 tiles on a grid of one round).  Each tile is split into PT row
// bands of one 16-byte word per lane; workgroup b takes band lr % PT of tile
// u = lr / PT, lr = xcd_logical_id(b, n):
// the GEMM wrote every slab of tile u from the workgroups of one XCD (split
// fastest, each XCD a contiguous range of logical ids), and when the number
// of tiles is a multiple of 8 that XCD is the one this workgroup runs on, so
// the slabs are still in its L2 (lines written by an XCD stay valid in its
// L2 across the kernel boundary).  Any other count only loses locality.
// Needs N % 4 == 0, so that 16-byte words never straddle a row or the edge
// of a column tile.  Same arithmetic as the flat pass: ascending s, F32.
template <int S, int BM, int BN, int OT>
__global__ __launch_bounds__(kBlock) void slab_reduce_tiles(const float* __restrict__ P,
                                                            void* __restrict__ C, int M, int N,
                                                            int tiles_m, FastDiv by_tiles_m) {
    constexpr int C4 = BN / 4;                  // 16-byte words per tile row
    constexpr int PT = tile_bands(BM, BN);      // workgroups per tile
    constexpr int ITEMS = BM * C4 / PT / kBlock;  // words per lane
    static_assert(ITEMS >= 1 && BM * C4 % (PT * kBlock) == 0, "tile size");
    const int lr = xcd_logical_id(blockIdx.x, gridDim.x);
    const int u = lr / PT, band = lr % PT;
    const int nt = (int)fastdiv((uint32_t)u, by_tiles_m), mt = u - nt * tiles_m;
    const int valid4 = min(C4, (N - nt * BN) / 4);  // words of a tile row inside N
    const int64_t plane = (int64_t)M * N;
    const float* tile = P + ((int64_t)mt * BM + band * (BM / PT)) * N + (int64_t)nt * BN;
    f32x4 v[ITEMS][S];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int i = threadIdx.x + it * kBlock;
        const int row = i / C4, c4 = i % C4;
        if (c4 < valid4) {
#pragma unroll
            for (int s = 0; s < S; ++s) v[it][s] = *(const f32x4*)(tile + s * plane + (int64_t)row * N + 4 * c4);
        }
    }
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int i = threadIdx.x + it * kBlock;
        const int row = i / C4, c4 = i % C4;
        if (c4 < valid4) {
            f32x4 acc = v[it][0];
#pragma unroll
            for (int s = 1; s < S; ++s) acc += v[it][s];
            store4<OT>(C, (((int64_t)mt * BM + band * (BM / PT) + row) * N + (int64_t)nt * BN) / 4 + c4, acc);
        }
    }
}

template <int S, int BM, int BN, int OT>
hipError_t launch_tiles(const float* partials, void* C, int64_t M, int64_t N, hipStream_t stream) {
    const int tiles_m = (int)(M / BM), tiles_n = (int)((N + BN - 1) / BN);
    int m = (int)M, n = (int)N, tm = tiles_m;
    FastDiv by_tm = make_fastdiv((uint32_t)tiles_m);
    void* args[] = {(void*)&partials, &C, &m, &n, &tm, &by_tm};
    return hipLaunchKernel((const void*)&slab_reduce_tiles<S, BM, BN, OT>,
                           dim3((unsigned)(tiles_m * tiles_n * tile_bands(BM, BN))), dim3(kBlock), args, 0,
                           stream);
}

template <int BM, int BN, int OT>
hipError_t launch_tiles_s(const float* partials, void* C, int s, int64_t M, int64_t N, hipStream_t st) {
    switch (s) {
        case 1: return launch_tiles<1, BM, BN, OT>(partials, C, M, N, st);
        case 2: return launch_tiles<2, BM, BN, OT>(partials, C, M, N, st);
        case 3: return launch_tiles<3, BM, BN, OT>(partials, C, M, N, st);
        case 4: return launch_tiles<4, BM, BN, OT>(partials, C, M, N, st);
        case 5: return launch_tiles<5, BM, BN, OT>(partials, C, M, N, st);
        case 6: return launch_tiles<6, BM, BN, OT>(partials, C, M, N, st);
        case 7: return launch_tiles<7, BM, BN, OT>(partials, C, M, N, st);
        case 8: return launch_tiles<8, BM, BN, OT>(partials, C, M, N, st);
        default: return hipErrorInvalidValue;
    }
}

template <int OT>
hipError_t launch_tiles_out(int bm, int bn, const float* partials, void* C, int s, int64_t M, int64_t N,
                            hipStream_t st) {
    if (bm == 32 && bn == 32) return launch_tiles_s<32, 32, OT>(partials, C, s, M, N, st);
    if (bm == 32 && bn == 64) return launch_tiles_s<32, 64, OT>(partials, C, s, M, N, st);
    if (bm == 64 && bn == 64) return launch_tiles_s<64, 64, OT>(partials, C, s, M, N, st);
    if (bm == 256 && bn == 128) return launch_tiles_s<256, 128, OT>(partials, C, s, M, N, st);
    if (bm == 256 && bn == 256) return launch_tiles_s<256, 256, OT>(partials, C, s, M, N, st);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_slab_reduce_after(const GemmPlan& plan, const float* partials, void* C,
                                    int64_t splits, int64_t M, int64_t N, int out_dtype,
                                    hipStream_t stream) {
    const bool tile_shape = (plan.bm == 32 && (plan.bn == 32 || plan.bn == 64)) ||
                            (plan.bm == 64 && plan.bn == 64) ||
                            (plan.bm == 256 && (plan.bn == 128 || plan.bn == 256));
    if (plan.order == 1 && tile_shape && splits <= 8 && N % 4 == 0 && M % plan.bm == 0) {
        const int s = (int)splits;
        switch (out_dtype) {
            case 0: return launch_tiles_out<0>(plan.bm, plan.bn, partials, C, s, M, N, stream);
            case 1: return launch_tiles_out<1>(plan.bm, plan.bn, partials, C, s, M, N, stream);
            case 2: return launch_tiles_out<2>(plan.bm, plan.bn, partials, C, s, M, N, stream);
            default: return hipErrorInvalidValue;
        }
    }
    return launch_slab_reduce(partials, C, splits, M, N, out_dtype, stream);
}

hipError_t launch_slab_reduce(const float* partials, void* C, int64_t splits, int64_t M, int64_t N,
                              int out_dtype, hipStream_t stream) {
    const int64_t plane4 = M * N / 4;
    const int s = (int)splits;
    switch (out_dtype) {
        case 0: return launch_out<0>(partials, C, s, plane4, stream);
        case 1: return launch_out<1>(partials, C, s, plane4, stream);
        case 2: return launch_out<2>(partials, C, s, plane4, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace splitk
