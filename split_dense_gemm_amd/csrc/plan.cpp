// Kernel choice for a validated problem: the shape rules, the tile order,
// the persistent form, named configurations, and the grid a plan launches.
// Host code only; the kernels and their launchers are in gemm_bt.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "splitk_internal.h"

namespace splitk {

// Compute units of the current device, looked up once per device.
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// A named configuration (tests and tuning sweeps, through
// splitk_gemm_planned): "wavek,BM,BN,WAVES,STAGES", "wavekdma,BM,BN,WAVES,
// REGCHUNKS" or "tiled,BM,BN,WM,WN[,RING]" (RING: LDS chunk buffers, default
// the tile's own).  True if the text names an instantiated configuration
// for this layout of B; *kind and v[0..4] then describe it.
static bool parse_plan(const char* text, int layout, int* kind, int* v) {
    char name[16] = {0};  // "wavek", "wavekdma", "tiled" or "tiledp"
    v[4] = 0;
    v[5] = 0;
    const int got = text ? sscanf(text, "%15[a-z],%d,%d,%d,%d,%d", name, &v[0], &v[1], &v[2], &v[3], &v[4]) : 0;
    if (got != 5 && got != 6) return false;
    if (!strcmp(name, "wavek") && got == 5 && wavek_config_exists(layout, v[0], v[1], v[2], v[3])) {
        *kind = kWaveK;
        return true;
    }
    if (!strcmp(name, "wavekdma") && got == 5 && layout == kLayoutNK &&
        wavekdma_config_exists(v[0], v[1], v[2], v[3])) {
        *kind = kWaveKDma;
        return true;
    }
    if (!strcmp(name, "tiled")) {
        if (got == 5) v[4] = tiled_nbuf(v[0], v[1]);
        if (tiled_config_exists(layout, v[0], v[1], v[2], v[3], v[4])) { *kind = kTiled; return true; }
    }
    if (!strcmp(name, "tiledp") && got == 5 && tiled_pt_config_exists(layout, v[0], v[1], v[2], v[3])) {
        v[4] = 2;
        v[5] = 1;
        *kind = kTiled;
        return true;
    }
    return false;
}

// The configuration the shape rules pick.
static GemmPlan plan_by_shape(int dtype, int64_t M, int64_t N, int64_t K, int64_t kps,
                              int64_t splits, int layout) {
    (void)K;
    const int64_t es = dtype == 0 ? 4 : 2;
    const int64_t ck = 128 / es;  // elements per 128-byte chunk
    const int64_t max_chunks = (kps + ck - 1) / ck;  // chunks of the longest split
    auto cdiv = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
    // Large problems: 256x256 tiles (2x2 waves) when there is at least one
    // per CU, else 256x128 tiles on 2x4 waves (two waves per SIMD, measured
    // 5-8% faster than 2x2 for this tile); these read the least L2 data per
    // flop.  For 16-bit inputs an N that 256 does not divide counts its
    // narrowed last column tile as a whole one and follows the same rules:
    // over twelve such shapes (N 2000-8000, N mod 256 from 8 to 216, 2-8
    // splits) 256x256 tiles ran the chain at 0.87-1.02x the 256x128 time
    // with B as [N,K] where the rules below pick them (0.97x at geometric
    // mean; 0.99-1.04x on the three half-full last rounds that they leave
    // to 256x128 tiles), and at 0.80-0.97x with B as [K,N].
    //
    // With B as [N,K], 256x128 tiles also take over where the last round of
    // 256x256 ones would be at most half full (workgroups mod 256 CUs in
    // 1..128): twice the workgroups at half the work each end half a round
    // earlier.  F32, GEMM + sum: 0.78x at 288 workgroups (2048x4608x4096 in
    // two splits 973.5 -> 757.5 us), 0.85-0.88x at 576, 0.93x at 1152; on
    // whole rounds 256x256 stays 1-7% faster.  16-bit inputs gain less:
    // BF16 0.87-0.90x at 257-384 workgroups in one or two splits
    // (4096x4608x4096 in one split 172.0 -> 149.9 us, 3072x6144x1536
    // 80.6 -> 69.5), F16 0.90-0.91x; further out only with short splits,
    // since long ones reverse it (3072x6144x12288 in four splits, 1152
    // workgroups: 452.6 -> 527.9 us) and the split-count model ranks such
    // 256x128 plans of many splits too cheaply.  So 16-bit inputs switch in
    // one or two splits up to 384 workgroups, or with at most 12 chunks per
    // split.  Over 200 BF16 (shape, split) pairs this takes the time from
    // 1.049 to 1.011x the faster of the two tiles at geometric mean.  With
    // B as [K,N] the 256x128 kernel was 3-7% slower on four such grids, and
    // 256x256 stays.
    // F32: the large tiles run at the F32 MFMA rate and are bound by MFMA
    // time rather than by staging, so the tile that packs the rounds best
    // wins: the fewest rounds x tile area x a per-tile factor (256x256 1,
    // 256x128 1.05, 128x128 1.1; ties to the larger tile; B as [K,N] has no
    // 128x128 kernel).  Over 68 F32 shapes and splits the large-tile rules
    // sent to 256x256 or 256x128 tiles (M 1024-3072, N 1536-6144, K 2048 and
    // 8192, 1-4 splits, B as [N,K]), each timed with all three tiles, this
    // picks the fastest every time: 0.91x the earlier choice at geometric
    // mean, 0.79x at best (2048x4608x8192 in one split on 128x128 tiles:
    // 1951 -> 1546 us).  B as [K,N], 256x128 against 256x256: 0.79-0.89x on
    // grids of 288-576 256x256 workgroups, 1.04x on a whole round of 512.
    const bool large = M % 256 == 0 && ((N % 256 == 0 && (M / 256) * (N / 256) * splits >= 256) ||
                                        (M / 256) * cdiv(N, 128) * splits >= 256);
    if (large && dtype == 0) {
        struct Tile { int bm, bn, wm, wn; double factor; };
        const Tile tiles[] = {{256, 256, 2, 2, 1.0}, {256, 128, 2, 4, 1.05}, {128, 128, 2, 2, 1.1}};
        const Tile* best = nullptr;
        int64_t best_wg = 0;
        double best_cost = 0.0;
        for (const Tile& t : tiles) {
            if (t.bn == 256 && N % 256 != 0) continue;
            if (t.bm == 128 && layout != kLayoutNK) continue;
            const int64_t wg = (M / t.bm) * cdiv(N, t.bn) * splits;
            const double cost = (double)((wg + 255) / 256) * t.bm * t.bn * t.factor;
            if (!best || cost < best_cost * (1.0 - 1e-9)) { best = &t; best_wg = wg; best_cost = cost; }
        }
        return GemmPlan{kTiled, best->bm, best->bn, best->wm * best->wn, best->wm, best_wg,
                        best->wm * best->wn * 64, layout, tiled_nbuf(best->bm, best->bn)};
    }
    if (M % 256 == 0 && (M / 256) * cdiv(N, 256) * splits >= 256) {
        const int64_t wg = (M / 256) * cdiv(N, 256) * splits;
        const bool half_round = wg % 256 != 0 && wg % 256 <= 128;
        const bool short_last_round =
            layout == kLayoutNK && half_round &&
            (dtype == 0 || (splits <= 2 && wg <= 384) || max_chunks <= 12);
        if (!short_last_round)
            return GemmPlan{kTiled, 256, 256, 4, 2, wg, 256, layout, tiled_nbuf(256, 256)};
    }
    if (M % 256 == 0 && (M / 256) * cdiv(N, 128) * splits >= 256)
        return GemmPlan{kTiled, 256, 128, 8, 2, (M / 256) * cdiv(N, 128) * splits, 512, layout,
                        tiled_nbuf(256, 128)};
    // Skinny problems.  Tile: the one that moves the fewest bytes through
    // the busiest CU.  Each workgroup streams (BM + BN) rows of its split,
    // and workgroups beyond the 256 CUs queue behind the first round.
    struct Cand { int bm, bn; };
    const Cand cands[] = {{32, 64}, {32, 32}};
    int bm = 32, bn = 32;
    int64_t best_cost = -1;
    for (const Cand& c : cands) {
        if (M % c.bm) continue;
        const int64_t wg = (M / c.bm) * cdiv(N, c.bn) * splits;
        const int64_t cost = ((wg + 255) / 256) * (c.bm + c.bn) * kps * es;
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; bm = c.bm; bn = c.bn; }
    }
    // Waves and stages: eight waves per workgroup (two per SIMD) measured
    // best at every shape of this family; enough register stages to keep a
    // wave's whole share of the split in flight, up to two.
    const int64_t chunks = max_chunks;
    const int w = 8;
    const int64_t wg = (M / bm) * cdiv(N, bn) * splits;
    // Each wave's last chunk by LDS DMA whenever a wave has at most two.
    const int64_t per_wave = (chunks + w - 1) / w;
    if (layout == kLayoutNK && per_wave <= 2 && wavekdma_config_exists(bm, bn, w, (int)per_wave - 1))
        return GemmPlan{kWaveKDma, bm, bn, w, (int)per_wave - 1, wg, w * 64, layout};
    int d = per_wave >= 2 ? 2 : 1;
    while (d > 1 && !wavek_config_exists(layout, bm, bn, w, d)) d /= 2;
    return GemmPlan{kWaveK, bm, bn, w, d, wg, w * 64, layout};
}

// Operand bytes one XCD may stream for the tiles it holds at once under the
// split-fastest order (order 1): past this the K range of those tiles
// crowds the 4 MiB L2.  Measured: 1.5 MiB (256x1024x2048, 2 splits) and
// 2.25 MiB (512x1024x2048, 2 splits) gain 0.35 and 1.3 us per GEMM + slab
// sum; 4.5 MiB (64x768x12288, 8 splits; 192x768x6144, 2 splits) and more
// lost 0.4-11 us, the GEMM slowing by up to 27%.
constexpr int64_t kSplitFastBytes = int64_t(3) << 20;

// Slabs of a large-tile GEMM up to this size stay in the L2s of the eight
// XCDs (4 MiB each) until the slab sum reads them.
constexpr int64_t kTiledLocalSlabBytes = int64_t(32) << 20;

// Tile order of a plan: split fastest where the tile-ordered slab sum
// applies (2..8 splits, N % 4 == 0) and
//  - for a skinny tile (32x32, 32x64, 64x64), the operand panels of the
//    tiles on one XCD fit kSplitFastBytes;
//  - for a large tile (256x128, 256x256), the grid is one round, the slabs
//    fit kTiledLocalSlabBytes and a split is at most 12 chunks of K.
//    Summing every slab on the XCD that wrote it then also spares the next
//    GEMM, a gain of a few microseconds, while the GEMM loses the panels the
//    split-major order shares on an XCD, a loss that grows with the split
//    length.  Measured with 256x128 tiles, GEMM + sum: 3 to 12 chunks
//    0.65-1.04x the split-major time (20.1 -> 15.9 us for 768x1536x1536 in
//    4 splits, 22.7 -> 14.7 for 512x1536x1536 in 8), 24 chunks and more
//    0.96-1.13x (28.2 -> 31.7 for 768x768x12288 in 8 splits); past one
//    round 34.9 -> 38.3 (1536x1536x3072, 4 splits, 288 workgroups).
static int tile_order(const GemmPlan& p, int dtype, int64_t M, int64_t N, int64_t K, int64_t kps,
                      int64_t splits) {
    if (splits < 2 || splits > 8 || N % 4 != 0) return 0;
    const int64_t es = dtype == 0 ? 4 : 2;
    if (p.kind == kTiled) {
        if (!(p.bm == 256 && (p.bn == 128 || p.bn == 256))) return 0;
        const int64_t chunks = (kps * es + 127) / 128;
        return p.grid <= device_cus() && splits * M * N * 4 <= kTiledLocalSlabBytes && chunks <= 12
                   ? 1 : 0;
    }
    if (!((p.bm == 32 && (p.bn == 32 || p.bn == 64)) || (p.bm == 64 && p.bn == 64))) return 0;
    const int64_t tiles_m = M / p.bm;
    const int64_t held = 32 / splits > 1 ? 32 / splits : 1;  // tiles per XCD at once, one workgroup per CU
    const int64_t rows = (held < tiles_m ? held : tiles_m) * p.bm + ((held + tiles_m - 1) / tiles_m) * p.bn;
    return rows * K * es <= kSplitFastBytes ? 1 : 0;
}

GemmPlan plan_gemm(int dtype, int64_t M, int64_t N, int64_t K, int64_t kps, int64_t splits,
                   int layout) {
    GemmPlan p = plan_by_shape(dtype, M, N, K, kps, splits, layout);
    // With too few 256-row tiles to fill the chip the rules above pick a
    // skinny kernel, but where M allows 256-row tiles the large-tile kernel
    // can still be faster on fewer CUs: each of its workgroups streams about
    // a third of the bytes per flop.  Take whichever the cost model of the
    // split-count choice rates faster.
    if (p.kind != kTiled && M % 256 == 0) {
        const int64_t tiles = (M / 256) * ((N + 127) / 128) * splits;
        const GemmPlan big{kTiled, 256, 128, 8, 2, tiles, 512, layout, tiled_nbuf(256, 128)};
        if (gemm_cost_us(big, dtype, M, N, K, kps, splits) < gemm_cost_us(p, dtype, M, N, K, kps, splits))
            p = big;
    }
    p.order = tile_order(p, dtype, M, N, K, kps, splits);
    // Grids of several rounds of 256x256 tiles, splits of at most 16 chunks:
    // the persistent kernel, which starts each CU's next tile while the last
    // one's partials are still being stored.  Measured on BF16 2048x4096 at
    // 8 splits against the one-tile kernel, B as [N,K]: 0.92x at 4 chunks
    // per split, 0.94-0.97x at 8 (the 2048x4096x4096 workload), 0.98x at 16,
    // 1.01x at 32; 4096x4096x4096 at 8 splits 0.98x, F16 0.97x, F32 0.99x.
    // B as [K,N], GEMM alone: 0.93x at 4 chunks (2048x4096x2048 in 8
    // splits), 0.96-0.97x at 8 (2048x4096x4096, 2048x4000x4096,
    // 4096x4096x4096 in 8 splits), 0.98-1.00x at 16.
    const int64_t es = dtype == 0 ? 4 : 2;
    if (p.kind == kTiled && p.bm == 256 && p.bn == 256 && p.waves == 4 && p.stages == 2 &&
        p.order == 0 && p.grid > device_cus() && (kps * es + 127) / 128 <= 16)
        p.persist = 1;
    return p;
}

bool plan_gemm_named(const char* text, int dtype, int64_t M, int64_t N, int64_t K, int64_t kps,
                     int64_t splits, int layout, GemmPlan* out) {
    int kind, f[6];
    if (!parse_plan(text, layout, &kind, f) || M % f[0] != 0) return false;
    const int64_t es = dtype == 0 ? 4 : 2;
    const int64_t max_chunks = (kps * es + 127) / 128;  // chunks of the longest split
    // The DMA-tail kernel holds at most waves x (register chunks + 1) chunks.
    if (kind == kWaveKDma && max_chunks > (int64_t)f[2] * (f[3] + 1)) return false;
    const int64_t wg = (M / f[0]) * ((N + f[1] - 1) / f[1]) * splits;
    GemmPlan p = kind == kTiled ? GemmPlan{kTiled, f[0], f[1], f[2] * f[3], f[2], wg, f[2] * f[3] * 64, layout, f[4]}
                                : GemmPlan{kind, f[0], f[1], f[2], f[3], wg, f[2] * 64, layout};
    p.order = tile_order(p, dtype, M, N, K, kps, splits);
    if (f[5]) {
        // Persistent: split-major order; every XCD needs a workgroup.
        if (wg < 8) return false;
        p.persist = 1;
        p.order = 0;
    }
    *out = p;
    return true;
}

// Workgroups a plan launches: the persistent kernel runs at most one per CU
// (a multiple of 8, so that every XCD has one), the others one per tile.
int64_t launch_grid(const GemmPlan& p) {
    if (!p.persist) return p.grid;
    const int64_t cap = std::max(8, device_cus() & ~7);
    return p.grid < cap ? p.grid : cap;
}

}  // namespace splitk
