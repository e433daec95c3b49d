// Split-count choice: the (k_per_split, splits) pair with the lowest
// modelled time for the whole operation, GEMM plus accumulation pass.
//
// The pages sample the split counts 1, 2, 4, 8 and 16 per shape and keep the
// fastest one ("Aligned shared rows for pipelined NAX on CUDA", section
// "Measurement protocol"; "Wider consecutive-weight NAX GEMM", section
// "Performance method").  Here the same candidates are ranked by a cost
// model of this library's own kernels on one 256-CU MI355X, so that no timing
// runs at call time:
//
//   GEMM    rounds * (a + b * staged MB per workgroup) + t0, floored by the
//           HBM time of its unique traffic, where rounds = workgroups /
//           (256 CUs * workgroups resident per CU), rounded up;
//   reduce  r0 + bytes moved / bandwidth (+ one more load round past eight
//           slabs); absent when one split writes C directly.
//
// The coefficients are least-squares fits to measured MI355X times of every
// (kernel family, element size) over 200 BF16 and 45 F32 shapes
// (M 32..4096, N 512..8192, K 1024..16384).  Candidates that are not powers of two
// (3, 6, 12) never won in those measurements and are not considered.
#include <math.h>
#include <stdint.h>

#include "splitk_internal.h"

namespace splitk {
namespace {

constexpr double kCus = 256.0;
constexpr double kHbmBytesPerUs = 5.5e6;   // sustained HBM3E rate, bytes per microsecond
constexpr double kHbmFloorUs = 1.0;
constexpr double kReduceBaseUs = 1.7;      // launch and one load round trip
constexpr double kReduceUsPerMB = 0.156;   // about 6.4 TB/s
constexpr double kReduceExtraRoundUs = 1.8;  // more than eight slabs: a second batch of loads

struct Coef {
    double t0, a, b;  // microseconds; b per MB staged by one workgroup
};

// [element size 2 or 4][family]: skinny with DMA tail, skinny, tiled 256x128, tiled 256x256.
constexpr Coef kCoef16[4] = {{0.57, 2.07, 10.65}, {0.04, 2.49, 11.84}, {3.90, 3.90, 22.60},
                             {0.91, 10.67, 28.71}};
constexpr Coef kCoef32[4] = {{0.20, 2.39, 23.72}, {-2.39, 4.52, 23.00}, {3.85, 3.85, 87.00},
                             {1.64, 10.39, 122.15}};

// Workgroups of one configuration resident on a CU at once, from each
// kernel's LDS use (160 KiB per CU) and VGPR use (512 per lane per SIMD).
// The same for all three element types.
int resident_per_cu(const GemmPlan& p) {
    if (p.kind == kTiled) return 1;
    if (p.kind == kWaveKDma) return (p.bn == 32 && p.stages == 0) ? 2 : 1;
    if (p.waves == 8) return (p.bn == 32 && p.stages == 1) ? 2 : 1;
    // Four-wave skinny configurations (reachable only through the override).
    if (p.bm == 32 && p.bn == 32) return p.stages <= 2 ? 4 : 2;
    if (p.bm == 32 && p.bn == 64) return p.stages == 1 ? 3 : (p.stages == 2 ? 2 : 1);
    return p.stages <= 2 ? 2 : 1;
}

const Coef& coef_of(const GemmPlan& p, int64_t es) {
    const Coef* table = es == 2 ? kCoef16 : kCoef32;
    if (p.kind == kWaveKDma) return table[0];
    if (p.kind == kWaveK) return table[1];
    return (p.bm == 256 && p.bn == 256) ? table[3] : table[2];
}

}  // namespace

double gemm_cost_us(const GemmPlan& p, int dtype, int64_t M, int64_t N, int64_t K, int64_t kps,
                    int64_t splits) {
    const int64_t es = dtype == 0 ? 4 : 2;
    const double rounds = ceil((double)p.grid / (kCus * resident_per_cu(p)));
    const double staged_mb = (double)(p.bm + p.bn) * (double)kps * (double)es / 1e6;
    const Coef& c = coef_of(p, es);
    const double t = c.t0 + rounds * (c.a + c.b * staged_mb);
    const double hbm = ((double)(M + N) * (double)K * es + (double)splits * M * N * 4) / kHbmBytesPerUs;
    return fmax(t, kHbmFloorUs + hbm);
}

double reduce_cost_us(int64_t splits, int64_t M, int64_t N, int out_dtype) {
    const double out_es = out_dtype == 0 ? 4.0 : 2.0;
    const double mb = ((double)splits * 4.0 + out_es) * (double)M * (double)N / 1e6;
    return kReduceBaseUs + kReduceUsPerMB * mb + (splits > 8 ? kReduceExtraRoundUs : 0.0);
}

int64_t split_length(int dtype, int64_t K, int64_t splits) {
    // Whole 128-byte chunks per split where that keeps every split starting
    // below K (no half chunk except possibly at the very end), else the
    // contract's 32-element granularity.
    const int64_t chunk = dtype == 0 ? 32 : 64;
    const int64_t even = (K + splits - 1) / splits;
    for (int64_t g : {chunk, (int64_t)32}) {
        const int64_t kps = (even + g - 1) / g * g;
        if ((splits - 1) * kps < K && splits * kps >= K) return kps;
    }
    return 0;
}

bool choose_split(int dtype, int out_dtype, int64_t M, int64_t N, int64_t K, int64_t* kps_out,
                  int64_t* splits_out) {
    static const int64_t kCandidates[] = {1, 2, 4, 8, 16};
    const int64_t max_elems = int64_t(1) << 31;
    double best = 0.0;
    bool found = false;
    for (int64_t s : kCandidates) {
        const int64_t kps = split_length(dtype, K, s);
        if (kps == 0 || s * (M * N) >= max_elems) continue;
        const GemmPlan p = plan_gemm(dtype, M, N, K, kps, s);
        double t = gemm_cost_us(p, dtype, M, N, K, kps, s);
        // One split writes an F32 C directly; any other case runs the pass.
        if (s > 1 || out_dtype != 0) t += reduce_cost_us(s, M, N, out_dtype);
        if (!found || t < best) {  // ties keep the smaller split count
            best = t;
            *kps_out = kps;
            *splits_out = s;
            found = true;
        }
    }
    return found;
}

}  // namespace splitk
