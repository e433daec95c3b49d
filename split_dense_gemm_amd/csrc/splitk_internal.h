// Internal interface between the C ABI (splitk_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace splitk {

// One chunk of K: 128 bytes of a row (8 pieces of 16 bytes).
constexpr int kChunkBytes = 128;

// Which GEMM kernel family serves a call.
enum GemmKind : int {
    // Skinny shapes (few output tiles): the W waves of a workgroup take the
    // split's 128-byte k-chunks round-robin, each staging its chunks through
    // registers and a private LDS area (`stages` chunks in flight), and their
    // partial tiles are summed through LDS in a fixed wave order.
    kWaveK = 0,
    // Large problems with enough tiles to fill the chip: a BM x BN tile per
    // workgroup whose WM x WN waves share every chunk, fed by LDS DMA through
    // a ring of LDS buffers (`stages` = waves along M).
    kTiled = 1,
    // As kWaveK, but each wave's last chunk travels by LDS DMA; for splits
    // short enough that a wave holds at most `stages` + 1 chunks.
    kWaveKDma = 2,
};

// Storage of B: [N,K] (each row k-contiguous) or [K,N] (each row n-contiguous).
enum BLayout : int { kLayoutNK = 0, kLayoutKN = 1 };

struct GemmPlan {
    int kind;
    int bm, bn, waves, stages;  // tiled kernels: stages = waves along M
    int64_t grid;  // workgroups
    int block;     // threads per workgroup
    int layout;    // BLayout of B
    int nbuf = 0;  // tiled kernels: chunk buffers in the LDS ring (0: the tile's default)
    int order = 0; // 1 = splits of a tile on one XCD (skinny_tile; the large-tile kernel's tile order)
    int persist = 0; // tiled kernels: one workgroup per CU walking several tiles
};

// Renumbers workgroups so that consecutive logical ids run on one XCD.
// Workgroup b is dispatched to XCD b % 8; logical ids [start_x, start_x+cnt_x)
// go to XCD x.  It is a bijection on [0, n) whatever the dispatch order.
__device__ __attribute__((always_inline)) inline int xcd_logical_id(int b, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = b & 7, slot = b >> 3;
    return x < r ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
}

// Division by a divisor known on the host: a multiply-high, an add and a
// shift (the round-up method of Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994), instead of the ~25
// instructions of a runtime division.  Exact for every numerator below 2^31
// and divisor in [1, 2^31): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, x / d = (mulhi(x, m) + x) >> l, and the
// sum stays below 2^32 because mulhi(x, m) < x.
struct FastDiv {
    uint32_t mul;
    uint32_t shift;
};
inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while (l < 31 && (uint32_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{(uint32_t)m, l};
}
__device__ __attribute__((always_inline)) inline uint32_t fastdiv(uint32_t x, FastDiv f) {
    return (__umulhi(x, f.mul) + x) >> f.shift;
}

// Output tile grid of a skinny GEMM launch (and of the slab sum that visits
// it in the same order): tile counts, split count and tile order, with their
// divisors prepared on the host.
struct TileGrid {
    int tiles_m, tiles_n, splits, order;
    FastDiv by_tiles_m, by_tiles_n, by_splits;
};
inline TileGrid make_tile_grid(int tiles_m, int tiles_n, int splits, int order) {
    return TileGrid{tiles_m, tiles_n, splits, order, make_fastdiv((uint32_t)tiles_m),
                    make_fastdiv((uint32_t)tiles_n), make_fastdiv((uint32_t)splits)};
}

// Slabs larger than this are written and read as streaming (nontemporal)
// accesses.  The memory-side cache holds 256 MiB: slabs that fit stay there
// between the GEMM and the slab sum, and normal accesses are faster
// (2048x4096x4096 with 4 splits, 128 MiB of slabs: 3.5% slower streamed);
// slabs that do not fit only evict the operands, and streaming them is
// faster (2048x4096x4096 with 8 splits, 256 MiB: the chain 15% faster).
constexpr int64_t kStreamSlabBytes = int64_t(192) << 20;
inline bool stream_slabs(int64_t splits, int64_t M, int64_t N) {
    return splits > 1 && splits * M * N * 4 > kStreamSlabBytes;
}

// Capacity of the library-owned slab array (static_slabs.hip): 16 Mi F32
// elements, 64 MiB per GPU.
constexpr int64_t kStaticSlabFloats = int64_t(16) << 20;

// Device address of that array on the current device, looked up on the
// first call per device (hipGetSymbolAddress) and cached; NULL if the
// lookup fails.
float* static_slabs();

// Default ring depth of a tile: as many buffers as fit in 160 KiB, up to four.
constexpr int tiled_nbuf(int bm, int bn) {
    return (160 * 1024) / ((bm + bn) * kChunkBytes) > 4 ? 4 : (160 * 1024) / ((bm + bn) * kChunkBytes);
}

// Compute units of the current device (looked up once per device).
int device_cus();

// Whether a kernel configuration is instantiated (the lists in gemm_bt.hip).
bool wavekdma_config_exists(int bm, int bn, int w, int r);
bool wavek_config_exists(int layout, int bm, int bn, int w, int d);
bool tiled_pt_config_exists(int layout, int bm, int bn, int wm, int wn);
bool tiled_config_exists(int layout, int bm, int bn, int wm, int wn, int nbuf);

// Chooses the kernel configuration for a validated problem.
GemmPlan plan_gemm(int dtype, int64_t M, int64_t N, int64_t K, int64_t kps, int64_t splits,
                   int layout = kLayoutNK);

// The instantiated configuration a plan text names (see splitk_gemm_planned
// in splitk.h), with the tile order plan_gemm would give it; false if the
// text names none for this layout of B, its row tile does not divide M, or
// (DMA-tail kernel) a split holds more chunks than its waves can take.
bool plan_gemm_named(const char* text, int dtype, int64_t M, int64_t N, int64_t K, int64_t kps,
                     int64_t splits, int layout, GemmPlan* out);

int64_t launch_grid(const GemmPlan& p);
hipError_t launch_gemm_bt(const GemmPlan& plan, const void* A, const void* B, float* partials,
                          int64_t M, int64_t N, int64_t K, int64_t kps, int64_t splits, int dtype,
                          hipStream_t stream);

// out_dtype: 0 F32, 1 F16, 2 BF16 (the sum is formed in F32, then rounded).
hipError_t launch_slab_reduce(const float* partials, void* C, int64_t splits, int64_t M, int64_t N,
                              int out_dtype, hipStream_t stream);

// The same sum for slabs that the GEMM `plan` has just written: after a
// GEMM in the split-fastest order (plan.order == 1) each workgroup takes one
// output tile, or one band of it, on the XCD whose L2 holds that tile's
// slabs; otherwise the flat pass above.
hipError_t launch_slab_reduce_after(const GemmPlan& plan, const float* partials, void* C,
                                    int64_t splits, int64_t M, int64_t N, int out_dtype,
                                    hipStream_t stream);

// Split-count choice (split_choice.cpp).  Modelled microseconds of one GEMM
// launch and of one accumulation pass on MI355X.
double gemm_cost_us(const GemmPlan& p, int dtype, int64_t M, int64_t N, int64_t K, int64_t kps,
                    int64_t splits);
double reduce_cost_us(int64_t splits, int64_t M, int64_t N, int out_dtype);
// k_per_split for `splits` even slices of K (0 if no valid geometry exists).
int64_t split_length(int dtype, int64_t K, int64_t splits);
// The candidate with the lowest modelled time; false if none is valid.
bool choose_split(int dtype, int out_dtype, int64_t M, int64_t N, int64_t K, int64_t* kps,
                  int64_t* splits);

}  // namespace splitk
