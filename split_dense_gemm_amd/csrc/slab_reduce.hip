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

// Store of one 16-byte F32 word as output type OT (0 F32, 1 F16, 2 BF16).
template <int OT>
__device__ inline void store4(void* C, int64_t g, f32x4 v) {
    if (OT == 0) {
        ((f32x4*)C)[g] = v;
    } else if (OT == 1) {
        ((f16x4*)C)[g] = __builtin_convertvector(v, f16x4);
    } else {
        ((bf16x4*)C)[g] = __builtin_convertvector(v, bf16x4);
    }
}

template <int S, int ITEMS, int OT>
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
                store4<OT>(C, g, acc);
            }
        }
    } else {
        // Any other split count: slabs in batches of eight whose loads are
        // all issued before their adds, still summed in ascending s.
        constexpr int kBatch = 8;
        for (int it = 0; it < ITEMS; ++it) {
            const int64_t g = g0 + it * stride;
            if (g >= plane4) break;
            f32x4 acc = P[g];
            int s = 1;
            for (; s + kBatch <= splits; s += kBatch) {
                f32x4 v[kBatch];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) v[j] = P[(int64_t)(s + j) * plane4 + g];
#pragma unroll
                for (int j = 0; j < kBatch; ++j) acc += v[j];
            }
            for (; s < splits; ++s) acc += P[(int64_t)s * plane4 + g];
            store4<OT>(C, g, acc);
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
    return hipLaunchKernel((const void*)&slab_reduce_kernel<S, ITEMS, OT>, grid, dim3(kBlock), args, 0,
                           stream);
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

}  // namespace

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
