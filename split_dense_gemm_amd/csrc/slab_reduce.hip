// Slab reduction: C[i,j] = sum over s of partials[s,i,j], in F32.
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

constexpr int kBlock = 256;

template <int S, int ITEMS>
__global__ __launch_bounds__(kBlock) void slab_reduce_kernel(const f32x4* __restrict__ P,
                                                             f32x4* __restrict__ C, int splits,
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
                for (int s = 0; s < S; ++s) v[it][s] = P[s * plane4 + g];
            }
        }
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t g = g0 + it * stride;
            if (g < plane4) {
                f32x4 acc = v[it][0];
#pragma unroll
                for (int s = 1; s < S; ++s) acc += v[it][s];
                C[g] = acc;
            }
        }
    } else {
        // Any other split count: ascending-s loop.
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t g = g0 + it * stride;
            if (g >= plane4) break;
            f32x4 acc = P[g];
            for (int s = 1; s < splits; ++s) acc += P[(int64_t)s * plane4 + g];
            C[g] = acc;
        }
    }
}

template <int S, int ITEMS>
hipError_t launch(const float* partials, float* C, int splits, int64_t plane4, hipStream_t stream) {
    const int64_t per_block = (int64_t)kBlock * ITEMS;
    const dim3 grid((unsigned)((plane4 + per_block - 1) / per_block));
    const f32x4* p = (const f32x4*)partials;
    f32x4* c = (f32x4*)C;
    void* args[] = {&p, &c, &splits, &plane4};
    return hipLaunchKernel((const void*)&slab_reduce_kernel<S, ITEMS>, grid, dim3(kBlock), args, 0,
                           stream);
}

template <int ITEMS>
hipError_t launch_items(const float* partials, float* C, int s, int64_t plane4, hipStream_t st) {
    switch (s) {
        case 1: return launch<1, ITEMS>(partials, C, s, plane4, st);
        case 2: return launch<2, ITEMS>(partials, C, s, plane4, st);
        case 3: return launch<3, ITEMS>(partials, C, s, plane4, st);
        case 4: return launch<4, ITEMS>(partials, C, s, plane4, st);
        case 5: return launch<5, ITEMS>(partials, C, s, plane4, st);
        case 6: return launch<6, ITEMS>(partials, C, s, plane4, st);
        case 7: return launch<7, ITEMS>(partials, C, s, plane4, st);
        case 8: return launch<8, ITEMS>(partials, C, s, plane4, st);
        default: return launch<0, ITEMS>(partials, C, s, plane4, st);
    }
}

}  // namespace

hipError_t launch_slab_reduce(const float* partials, float* C, int64_t splits, int64_t M, int64_t N,
                              hipStream_t stream) {
    const int64_t plane4 = M * N / 4;
    const int s = (int)splits;
    // Four words per lane once the plane gives every CU several workgroups
    // that way (measured faster for large planes); one word per lane
    // otherwise, so that small planes still spread over all CUs.
    if (plane4 >= (int64_t)256 * 4 * kBlock * 4)
        return launch_items<4>(partials, C, s, plane4, stream);
    return launch_items<1>(partials, C, s, plane4, stream);
}

}  // namespace splitk
