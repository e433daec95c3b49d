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
//   GEMM    t0 + rounds * (a + b * MB staged per wave + c * MB staged per
//           workgroup) + d * MB of partial slabs written, floored by the HBM
//           time of its unique traffic, where rounds = workgroups / (256 CUs
//           * workgroups resident per CU), rounded up.  In the skinny kernels
//           a wave's own chunk count sets the critical path (the waves of a
//           workgroup share the split's chunks); the large-tile kernels have
//           no per-wave term, but a slab term: each workgroup stores its
//           128-256 KiB tile after its last chunk with nothing to overlap,
//           and the store time grows with how many workgroups store at once,
//           which a per-round constant cannot follow;
//   reduce  r0 + bytes moved / bandwidth (+ one more load round past eight
//           slabs); absent when one split writes C directly.
//
// The coefficients are least-squares fits (relative error) to measured
// MI355X times of each (kernel family, element size): 480 BF16 shapes (M
// 32..4096, N 512..8192, K 1024..16384, including a dense grid of the small
// shapes M 32..320, N 512..1536, K 1024..6144) and 45 F32 shapes, each at
// all five split counts.  The large-tile rows are fitted on the whole
// operation instead (GEMM + slab sum, less the modelled sum), at all five
// split counts, each shape with the shape rules' kernel and with the 256x128
// kernel forced, which is where the families compete: 64 BF16 shapes (M 256,
// 512, 1024, 2048; N 768..6144; K 1536..12288) and 20 F32 shapes (M 32..2048,
// N 1024 and 4096, K 2048 and 8192).  Candidates that are not powers of two (3, 6, 12)
// never won in those measurements and are not considered.
#include <math.h>
#include <stdint.h>

#include "splitk_internal.h"

namespace splitk {
namespace {

constexpr double kCus = 256.0;
constexpr double kHbmBytesPerUs = 5.5e6;   // sustained HBM3E rate, bytes per microsecond
constexpr double kHbmFloorUs = 1.0;
constexpr double kReduceBaseUs = 1.95;       // launch gap and one load round trip
constexpr double kReduceUsPerMB = 0.157;      // about 6.4 TB/s
constexpr double kReduceExtraRoundUs = 2.29;  // more than eight slabs: a second batch of loads

struct Coef {
    double t0, a;  // microseconds
    double b;      // per MB staged by one wave (skinny kernels)
    double c;      // per MB staged by one workgroup
    double d;      // per MB of partial slabs written (large-tile kernels)
};

// [element size 2 or 4][family]: skinny with DMA tail, skinny, tiled 256x128,
// tiled 256x256, tiled 128x128.  The F32 128x128 row is fitted on 30 F32
// shapes (M 1024-3072, N 1536-6144, K 2048 and 8192) at 1, 2 and 4 splits;
// 16-bit inputs reach 128x128 tiles only through the override and are priced
// as 256x128.
constexpr Coef kCoef16[5] = {{0.701, 1.510, 62.80, 5.154, 0.0}, {-0.275, 2.723, 2.126, 11.14, 0.0},
                             {3.931, -1.702, 0.0, 14.46, 0.201}, {-0.844, 1.284, 0.0, 23.47, 0.136},
                             {3.931, -1.702, 0.0, 14.46, 0.201}};
constexpr Coef kCoef32[5] = {{0.543, 1.120, 140.1, 14.27, 0.0}, {-2.394, 4.521, 2.831, 22.65, 0.0},
                             {4.785, -0.551, 0.0, 76.71, 0.164}, {2.986, 0.0, 0.0, 114.4, 0.129},
                             {6.445, -5.188, 0.0, 61.02, 0.478}};

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
    if (p.bm == 128 && p.bn == 128) return table[4];
    return (p.bm == 256 && p.bn == 256) ? table[3] : table[2];
}

}  // namespace

double gemm_cost_us(const GemmPlan& p, int dtype, int64_t M, int64_t N, int64_t K, int64_t kps,
                    int64_t splits) {
    const int64_t es = dtype == 0 ? 4 : 2;
    const double rounds = ceil((double)p.grid / (kCus * resident_per_cu(p)));
    // Staged bytes: 128 per row of the BM + BN tile rows per chunk; a wave of
    // a skinny workgroup handles every waves-th chunk of the split.
    const int64_t chunks = (kps * es + 127) / 128;
    const double chunk_mb = (double)(p.bm + p.bn) * 128.0 / 1e6;
    const double per_wave = p.kind == kTiled ? 0.0 : (double)((chunks + p.waves - 1) / p.waves) * chunk_mb;
    const Coef& c = coef_of(p, es);
    const double slab_bytes = (double)splits * M * N * 4;
    const double t = c.t0 + rounds * (c.a + c.b * per_wave + c.c * (double)chunks * chunk_mb) +
                     c.d * slab_bytes / 1e6;
    const double hbm = ((double)(M + N) * (double)K * es + slab_bytes) / kHbmBytesPerUs;
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
