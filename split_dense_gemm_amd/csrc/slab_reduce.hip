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
// bound by memory bandwidth.  Each lane owns one 16-byte word of the [M*N]
// plane, issues all of its slab loads before the first add (so the loads of
// every slab are in flight together) and writes that word once; consecutive
// lanes touch consecutive words, so every load and store instruction of a
// wave covers 1 KiB of contiguous memory.  The
// slabs are read once and never again, so they are loaded non-temporally;
// the output is stored normally.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitk_internal.h"

namespace splitk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;

template <int MAXS>
__global__ __launch_bounds__(kBlock) void slab_reduce_kernel(const f32x4* __restrict__ P,
                                                             f32x4* __restrict__ C, int splits,
                                                             int64_t plane4) {
    const int64_t g = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (g >= plane4) return;
    if (MAXS > 0) {
        // Small split counts: every slab load issued up front.
        f32x4 v[MAXS > 0 ? MAXS : 1];
#pragma unroll
        for (int s = 0; s < MAXS; ++s)
            if (s < splits) v[s] = __builtin_nontemporal_load(P + (int64_t)s * plane4 + g);
        f32x4 acc = v[0];
#pragma unroll
        for (int s = 1; s < MAXS; ++s)
            if (s < splits) acc += v[s];
        C[g] = acc;
    } else {
        f32x4 acc = __builtin_nontemporal_load(P + g);
        for (int s = 1; s < splits; ++s) acc += __builtin_nontemporal_load(P + (int64_t)s * plane4 + g);
        C[g] = acc;
    }
}

template <int MAXS>
hipError_t launch(const float* partials, float* C, int splits, int64_t plane4, hipStream_t stream) {
    const dim3 grid((unsigned)((plane4 + kBlock - 1) / kBlock));
    const f32x4* p = (const f32x4*)partials;
    f32x4* c = (f32x4*)C;
    void* args[] = {&p, &c, &splits, &plane4};
    return hipLaunchKernel((const void*)&slab_reduce_kernel<MAXS>, grid, dim3(kBlock), args, 0, stream);
}

}  // namespace

hipError_t launch_slab_reduce(const float* partials, float* C, int64_t splits, int64_t M, int64_t N,
                              hipStream_t stream) {
    const int64_t plane4 = M * N / 4;
    const int s = (int)splits;
    if (s <= 2) return launch<2>(partials, C, s, plane4, stream);
    if (s <= 4) return launch<4>(partials, C, s, plane4, stream);
    if (s <= 8) return launch<8>(partials, C, s, plane4, stream);
    return launch<0>(partials, C, s, plane4, stream);
}

}  // namespace splitk
