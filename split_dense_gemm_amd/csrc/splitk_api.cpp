// C ABI of the split-K GEMM library: argument checks, kernel choice, launch.
//
// The checks restate the launch contract of "Aligned shared rows for
// pipelined NAX on CUDA" (section "Contract and correctness") and "Wider
// consecutive-weight NAX GEMM" (section "Launch contract and correctness"):
// M, K and k_per_split positive multiples of 32, every split starting below
// K with the splits covering K, exact extents and outputs that alias nothing.
// The pages also require N to be a multiple of 64; here any positive N is
// served (a narrowed last column tile), and a multiple of 8 when B is stored
// [K,N] so that its rows stay 16-byte aligned.  Each failed check returns its
// own status before anything is enqueued; no HIP call is made until every
// check has passed.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/splitk.h"
#include "splitk_internal.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 31;  // 32-bit element indices in the kernels

struct Range {
    uintptr_t lo, hi;  // [lo, hi) in bytes
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int element_bytes(int dtype) { return dtype == SPLITK_F32 ? 4 : 2; }

bool valid_dtype(int dtype) { return dtype == SPLITK_F32 || dtype == SPLITK_F16 || dtype == SPLITK_BF16; }

// N granularity per layout of B: any N for [N,K], multiples of 8 for [K,N].
int64_t n_multiple(int layout) { return layout == splitk::kLayoutKN ? 8 : 1; }

// Shape, split and size checks shared by the GEMM entry points.
int check_gemm_shape(int64_t M, int64_t N, int64_t K, int64_t kps, int64_t splits, int dtype,
                     int layout = splitk::kLayoutNK) {
    if (!valid_dtype(dtype)) return SPLITK_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K <= 0 || kps <= 0) return SPLITK_ERR_SHAPE;
    if (M % 32 || K % 32 || kps % 32 || N % n_multiple(layout)) return SPLITK_ERR_SHAPE;
    if (M >= kMaxElems || N >= kMaxElems || K >= kMaxElems || kps >= kMaxElems) return SPLITK_ERR_RANGE;
    // Every split starts below K and together they cover K.  With kps >= 32
    // any valid split count is below K, so the products below cannot overflow.
    if (splits < 1 || splits > K) return SPLITK_ERR_SPLIT;
    if ((splits - 1) * kps >= K || splits * kps < K) return SPLITK_ERR_SPLIT;
    if (M * K >= kMaxElems || N * K >= kMaxElems || M * N >= kMaxElems) return SPLITK_ERR_RANGE;
    if (splits * (M * N) >= kMaxElems) return SPLITK_ERR_RANGE;
    return SPLITK_OK;
}

// Pointer checks: alignment, then overlap of outputs with everything else.
// C may be NULL (GEMM alone); c_es is the byte size of one C element.
int check_gemm_pointers(const void* A, const void* B, const float* P, const void* C, int64_t M,
                        int64_t N, int64_t K, int64_t splits, int dtype, int64_t c_es) {
    if (!aligned16(A) || !aligned16(B) || !aligned16(P) || (C && !aligned16(C))) return SPLITK_ERR_ALIGN;
    const int64_t es = element_bytes(dtype);
    const Range ra{(uintptr_t)A, (uintptr_t)A + (uintptr_t)(M * K * es)};
    const Range rb{(uintptr_t)B, (uintptr_t)B + (uintptr_t)(N * K * es)};
    const Range rp{(uintptr_t)P, (uintptr_t)P + (uintptr_t)(splits * M * N * 4)};
    if (overlaps(rp, ra) || overlaps(rp, rb)) return SPLITK_ERR_ALIAS;
    if (C) {
        const Range rc{(uintptr_t)C, (uintptr_t)C + (uintptr_t)(M * N * c_es)};
        if (overlaps(rc, ra) || overlaps(rc, rb) || overlaps(rc, rp)) return SPLITK_ERR_ALIAS;
    }
    return SPLITK_OK;
}

int check_reduce(const float* P, const void* C, int64_t splits, int64_t M, int64_t N, int out_dtype) {
    if (!P || !C) return SPLITK_ERR_NULL;
    if (!valid_dtype(out_dtype)) return SPLITK_ERR_DTYPE;
    if (M <= 0 || N <= 0 || M % 32) return SPLITK_ERR_SHAPE;  // M*N is then a multiple of 4
    if (splits < 1) return SPLITK_ERR_SPLIT;
    if (M >= kMaxElems || N >= kMaxElems || splits >= kMaxElems) return SPLITK_ERR_RANGE;
    if (M * N >= kMaxElems || splits * (M * N) >= kMaxElems) return SPLITK_ERR_RANGE;
    if (!aligned16(P) || !aligned16(C)) return SPLITK_ERR_ALIGN;
    const Range rp{(uintptr_t)P, (uintptr_t)P + (uintptr_t)(splits * M * N * 4)};
    const Range rc{(uintptr_t)C, (uintptr_t)C + (uintptr_t)(M * N * element_bytes(out_dtype))};
    if (overlaps(rp, rc)) return SPLITK_ERR_ALIAS;
    return SPLITK_OK;
}

// Shape and type checks of the automatic-split entry points (no split
// geometry is given, so only the operands' own domain is checked).
int check_auto_shape(int64_t M, int64_t N, int64_t K, int dtype, int out_dtype) {
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return SPLITK_ERR_DTYPE;
    if (M <= 0 || N <= 0 || K <= 0 || M % 32 || K % 32) return SPLITK_ERR_SHAPE;
    if (M >= kMaxElems || N >= kMaxElems || K >= kMaxElems) return SPLITK_ERR_RANGE;
    if (M * K >= kMaxElems || N * K >= kMaxElems || M * N >= kMaxElems) return SPLITK_ERR_RANGE;
    return SPLITK_OK;
}

// F32 elements of workspace the automatic path needs: none when one split
// writes an F32 C directly, else the slabs.
int64_t auto_workspace(int64_t splits, int64_t M, int64_t N, int out_dtype) {
    return (splits == 1 && out_dtype == SPLITK_F32) ? 0 : splits * M * N;
}

// The library's kernel choice for a checked geometry, or the configuration
// `named` names (NULL: the library's choice).  False if the name is unknown
// or does not fit the problem.
bool pick_plan(const char* named, int layout, int dtype, int64_t M, int64_t N, int64_t K, int64_t kps,
               int64_t splits, splitk::GemmPlan* plan) {
    if (!named) {
        *plan = splitk::plan_gemm(dtype, M, N, K, kps, splits, layout);
        return true;
    }
    return splitk::plan_gemm_named(named, dtype, M, N, K, kps, splits, layout, plan);
}

// GEMM (and, when C is given, the accumulation pass) for either layout of B,
// with the library's kernel choice or a named one.
int gemm_entry(int layout, const void* A, const void* B, float* P, void* C, int64_t M, int64_t N,
               int64_t K, int64_t kps, int64_t splits, int dtype, int out_dtype, void* stream,
               const char* named = nullptr) {
    if (!A || !B || !P) return SPLITK_ERR_NULL;
    int st = check_gemm_shape(M, N, K, kps, splits, dtype, layout);
    if (st != SPLITK_OK) return st;
    if (C && !valid_dtype(out_dtype)) return SPLITK_ERR_DTYPE;
    st = check_gemm_pointers(A, B, P, C, M, N, K, splits, dtype, C ? element_bytes(out_dtype) : 0);
    if (st != SPLITK_OK) return st;
    splitk::GemmPlan plan;
    if (!pick_plan(named, layout, dtype, M, N, K, kps, splits, &plan)) return SPLITK_ERR_PLAN;
    hipError_t e = splitk::launch_gemm_bt(plan, A, B, P, M, N, K, kps, splits, dtype, (hipStream_t)stream);
    if (e != hipSuccess) return SPLITK_ERR_LAUNCH;
    if (C) e = splitk::launch_slab_reduce_after(plan, P, C, splits, M, N, out_dtype, (hipStream_t)stream);
    return e == hipSuccess ? SPLITK_OK : SPLITK_ERR_LAUNCH;
}

int describe_plan(int layout, int64_t M, int64_t N, int64_t K, int64_t k_per_split, int64_t splits,
                  int dtype, char* buf, int64_t len, const char* named = nullptr) {
    int st = check_gemm_shape(M, N, K, k_per_split, splits, dtype, layout);
    if (st != SPLITK_OK) return st;
    splitk::GemmPlan p;
    if (!pick_plan(named, layout, dtype, M, N, K, k_per_split, splits, &p)) return SPLITK_ERR_PLAN;
    if (buf && len > 0) {
        if (p.kind == splitk::kTiled)
            snprintf(buf, (size_t)len, "tiled bm%d bn%d waves%dx%d ring%d block%d grid%lld%s%s", p.bm, p.bn,
                     p.stages, p.waves / p.stages, p.nbuf, p.block, (long long)splitk::launch_grid(p),
                     p.order == 1 ? " splitfast" : "", p.persist ? " persistent" : "");
        else
            snprintf(buf, (size_t)len, "%s bm%d bn%d waves%d stages%d block%d grid%lld%s",
                     p.kind == splitk::kWaveKDma ? "wavekdma" : "wavek", p.bm, p.bn, p.waves, p.stages,
                     p.block, (long long)p.grid, p.order == 1 ? " splitfast" : "");
    }
    return SPLITK_OK;
}

}  // namespace

extern "C" {

const char* splitk_status_str(int status) {
    switch (status) {
        case SPLITK_OK: return "ok";
        case SPLITK_ERR_NULL: return "null pointer";
        case SPLITK_ERR_DTYPE: return "unknown dtype";
        case SPLITK_ERR_SHAPE:
            return "bad shape: M, K and k_per_split must be positive multiples of 32 and N positive "
                   "(a multiple of 8 when B is stored [K,N])";
        case SPLITK_ERR_SPLIT:
            return "bad split geometry: every split must start below K and the splits must cover K";
        case SPLITK_ERR_ALIAS: return "an output overlaps an input or the other output";
        case SPLITK_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case SPLITK_ERR_RANGE: return "a buffer holds 2^31 elements or more";
        case SPLITK_ERR_LAUNCH: return "kernel launch failed";
        case SPLITK_ERR_WORKSPACE:
            return "workspace smaller than the chosen split geometry needs (see splitk_choose_splits)";
        case SPLITK_ERR_SCRATCH:
            return "the chosen split geometry needs more slab memory than the library's static array "
                   "holds (16 Mi F32 elements; use splitk_gemm_bt_auto with a workspace)";
        case SPLITK_ERR_PLAN:
            return "the named kernel configuration is not instantiated for this layout of B or does not "
                   "fit the problem";
        default: return "unknown status";
    }
}

int splitk_gemm_bt(const void* A, const void* B, float* partials, int64_t M, int64_t N, int64_t K,
                   int64_t k_per_split, int64_t splits, int dtype, void* stream) {
    return gemm_entry(splitk::kLayoutNK, A, B, partials, nullptr, M, N, K, k_per_split, splits, dtype,
                      SPLITK_F32, stream);
}

int splitk_reduce_typed(const float* partials, void* C, int64_t splits, int64_t M, int64_t N,
                        int out_dtype, void* stream) {
    int st = check_reduce(partials, C, splits, M, N, out_dtype);
    if (st != SPLITK_OK) return st;
    hipError_t e = splitk::launch_slab_reduce(partials, C, splits, M, N, out_dtype, (hipStream_t)stream);
    return e == hipSuccess ? SPLITK_OK : SPLITK_ERR_LAUNCH;
}

int splitk_reduce(const float* partials, float* C, int64_t splits, int64_t M, int64_t N, void* stream) {
    return splitk_reduce_typed(partials, C, splits, M, N, SPLITK_F32, stream);
}

int splitk_reduce_for_gemm(const float* partials, void* C, int64_t M, int64_t N, int64_t K,
                           int64_t k_per_split, int64_t splits, int dtype, int out_dtype,
                           void* stream) {
    int st = check_reduce(partials, C, splits, M, N, out_dtype);
    if (st != SPLITK_OK) return st;
    st = check_gemm_shape(M, N, K, k_per_split, splits, dtype);
    if (st != SPLITK_OK) return st;
    const splitk::GemmPlan plan = splitk::plan_gemm(dtype, M, N, K, k_per_split, splits);
    hipError_t e = splitk::launch_slab_reduce_after(plan, partials, C, splits, M, N, out_dtype,
                                                    (hipStream_t)stream);
    return e == hipSuccess ? SPLITK_OK : SPLITK_ERR_LAUNCH;
}

int splitk_gemm_bt_reduce_typed(const void* A, const void* B, float* partials, void* C, int64_t M,
                                int64_t N, int64_t K, int64_t k_per_split, int64_t splits, int dtype,
                                int out_dtype, void* stream) {
    if (!C) return SPLITK_ERR_NULL;
    return gemm_entry(splitk::kLayoutNK, A, B, partials, C, M, N, K, k_per_split, splits, dtype,
                      out_dtype, stream);
}

int splitk_gemm_bt_reduce(const void* A, const void* B, float* partials, float* C, int64_t M,
                          int64_t N, int64_t K, int64_t k_per_split, int64_t splits, int dtype,
                          void* stream) {
    return splitk_gemm_bt_reduce_typed(A, B, partials, C, M, N, K, k_per_split, splits, dtype,
                                       SPLITK_F32, stream);
}

int splitk_choose_splits(int64_t M, int64_t N, int64_t K, int dtype, int out_dtype,
                         int64_t* k_per_split, int64_t* splits, int64_t* workspace_elems) {
    if (!k_per_split || !splits || !workspace_elems) return SPLITK_ERR_NULL;
    int st = check_auto_shape(M, N, K, dtype, out_dtype);
    if (st != SPLITK_OK) return st;
    int64_t kps = 0, s = 0;
    if (!splitk::choose_split(dtype, out_dtype, M, N, K, &kps, &s)) return SPLITK_ERR_RANGE;
    *k_per_split = kps;
    *splits = s;
    *workspace_elems = auto_workspace(s, M, N, out_dtype);
    return SPLITK_OK;
}

int splitk_gemm_bt_auto(const void* A, const void* B, float* workspace, int64_t workspace_elems,
                        void* C, int64_t M, int64_t N, int64_t K, int dtype, int out_dtype,
                        void* stream) {
    if (!A || !B || !C) return SPLITK_ERR_NULL;
    int64_t kps = 0, s = 0, need = 0;
    int st = splitk_choose_splits(M, N, K, dtype, out_dtype, &kps, &s, &need);
    if (st != SPLITK_OK) return st;
    if (workspace_elems < need) return SPLITK_ERR_WORKSPACE;
    const splitk::GemmPlan plan = splitk::plan_gemm(dtype, M, N, K, kps, s);
    if (need == 0) {
        // One split, F32 output: the GEMM's single slab is C itself.
        st = check_gemm_pointers(A, B, (const float*)C, nullptr, M, N, K, 1, dtype, 0);
        if (st != SPLITK_OK) return st;
        hipError_t e = splitk::launch_gemm_bt(plan, A, B, (float*)C, M, N, K, kps, 1, dtype,
                                              (hipStream_t)stream);
        return e == hipSuccess ? SPLITK_OK : SPLITK_ERR_LAUNCH;
    }
    if (!workspace) return SPLITK_ERR_NULL;
    st = check_gemm_pointers(A, B, workspace, C, M, N, K, s, dtype, element_bytes(out_dtype));
    if (st != SPLITK_OK) return st;
    hipError_t e = splitk::launch_gemm_bt(plan, A, B, workspace, M, N, K, kps, s, dtype,
                                          (hipStream_t)stream);
    if (e != hipSuccess) return SPLITK_ERR_LAUNCH;
    e = splitk::launch_slab_reduce_after(plan, workspace, C, s, M, N, out_dtype, (hipStream_t)stream);
    return e == hipSuccess ? SPLITK_OK : SPLITK_ERR_LAUNCH;
}

int splitk_gemm_bt_auto_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                                int dtype, int out_dtype, void* stream) {
    if (!A || !B || !C) return SPLITK_ERR_NULL;
    int64_t kps = 0, s = 0, need = 0;
    int st = splitk_choose_splits(M, N, K, dtype, out_dtype, &kps, &s, &need);
    if (st != SPLITK_OK) return st;
    if (need > splitk::kStaticSlabFloats) return SPLITK_ERR_SCRATCH;
    if (need == 0) {
        // One split, F32 output: the GEMM writes C itself, no slab memory.
        return splitk_gemm_bt_auto(A, B, nullptr, 0, C, M, N, K, dtype, out_dtype, stream);
    }
    float* slabs = splitk::static_slabs();
    if (!slabs) return SPLITK_ERR_LAUNCH;
    return splitk_gemm_bt_auto(A, B, slabs, splitk::kStaticSlabFloats, C, M, N, K, dtype, out_dtype, stream);
}

int splitk_describe(int64_t M, int64_t N, int64_t K, int64_t k_per_split, int64_t splits, int dtype,
                    char* buf, int64_t len) {
    return describe_plan(splitk::kLayoutNK, M, N, K, k_per_split, splits, dtype, buf, len);
}

int splitk_gemm_bn(const void* A, const void* B, float* partials, int64_t M, int64_t N, int64_t K,
                   int64_t k_per_split, int64_t splits, int dtype, void* stream) {
    return gemm_entry(splitk::kLayoutKN, A, B, partials, nullptr, M, N, K, k_per_split, splits, dtype,
                      SPLITK_F32, stream);
}

int splitk_gemm_bn_reduce(const void* A, const void* B, float* partials, void* C, int64_t M,
                          int64_t N, int64_t K, int64_t k_per_split, int64_t splits, int dtype,
                          int out_dtype, void* stream) {
    if (!C) return SPLITK_ERR_NULL;
    return gemm_entry(splitk::kLayoutKN, A, B, partials, C, M, N, K, k_per_split, splits, dtype,
                      out_dtype, stream);
}

int splitk_describe_bn(int64_t M, int64_t N, int64_t K, int64_t k_per_split, int64_t splits,
                       int dtype, char* buf, int64_t len) {
    return describe_plan(splitk::kLayoutKN, M, N, K, k_per_split, splits, dtype, buf, len);
}

int splitk_gemm_planned(const char* plan, int b_layout, const void* A, const void* B, float* partials,
                        void* C, int64_t M, int64_t N, int64_t K, int64_t k_per_split, int64_t splits,
                        int dtype, int out_dtype, void* stream) {
    if (!plan) return SPLITK_ERR_NULL;
    if (b_layout != splitk::kLayoutNK && b_layout != splitk::kLayoutKN) return SPLITK_ERR_PLAN;
    return gemm_entry(b_layout, A, B, partials, C, M, N, K, k_per_split, splits, dtype,
                      C ? out_dtype : SPLITK_F32, stream, plan);
}

int splitk_describe_planned(const char* plan, int b_layout, int64_t M, int64_t N, int64_t K,
                            int64_t k_per_split, int64_t splits, int dtype, char* buf, int64_t len) {
    if (!plan) return SPLITK_ERR_NULL;
    if (b_layout != splitk::kLayoutNK && b_layout != splitk::kLayoutKN) return SPLITK_ERR_PLAN;
    return describe_plan(b_layout, M, N, K, k_per_split, splits, dtype, buf, len, plan);
}

}  // extern "C"
