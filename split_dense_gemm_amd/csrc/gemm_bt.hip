// Split-K GEMM into F32 partial slabs for gfx950 (CDNA4).
//
// partials[s,i,j] = sum over k in [s*kps, min((s+1)*kps, K)) of A[i,k]*B[j,k]
// ("Aligned shared rows for pipelined NAX on CUDA", section "Contract and
// correctness"; "Wider consecutive-weight NAX GEMM", section "Launch contract
// and correctness").  A is [M,K] and k-contiguous; B is [N,K] (k-contiguous)
// or, for the [K,N] entry points, [K,N] (n-contiguous).
//
// The pages' own kernels (a 32x64 tile on 128 threads, 40-element padded
// shared rows, BF16 converted to F16 on the way in) were built for other
// hardware.  What is kept here is the contract.  The design is:
//
//  * Native MFMA on the stored element type: v_mfma_f32_32x32x16_{bf16,f16}
//    for 16-bit inputs and v_mfma_f32_32x32x2_f32 for F32, accumulating in
//    F32.  BF16 is never narrowed to F16.
//  * Work unit: a 128-byte k-chunk of every row of a BM x BN tile (BM rows of
//    A and BN rows of B).  Global loads are coalesced: each load instruction
//    of a wave reads eight whole 128-byte row segments; the transpose into
//    MFMA fragments happens in LDS, whose 16-byte slots are XOR-swizzled so
//    that the fragment reads are free of bank conflicts.  The order in which
//    an MFMA's k slots are filled does not change the dot product, so A and
//    B fragments only have to use the same slot -> k assignment.
//  * Three kernel families.  gemm_bt_wavek (skinny shapes): the waves of a
//    workgroup take the split's chunks round-robin through a register
//    pipeline and per-wave LDS staging, and their partial tiles are added
//    through LDS in a fixed wave order.  gemm_bt_wavek_dma: the same, with
//    each wave's last chunk loaded straight into LDS (global_load_lds).
//    gemm_bt_tiled (large problems): a 256-row tile whose waves share every
//    chunk, fed through a ring of LDS buffers by LDS DMA; gemm_bt_tiled_pt,
//    its persistent form for grids of several rounds, where each workgroup
//    walks several tiles and loads the next tile's first chunks while it
//    stores the last one's partials.  No atomics; every output element is
//    written once.
//  * Slice ends are multiples of 32 elements.  For 16-bit inputs a chunk is
//    64 elements, so the last chunk of a slice may be half empty: its loads
//    are redirected to in-bounds data of the same slice and its upper half
//    never reaches an MFMA (skipped steps or zeroed A fragments).  No load
//    touches memory past the operands' ends.
//  * Column tails: the last column tile may extend past N.  Its B rows past
//    N re-read row N-1 (or, for [K,N], the row's last 16 bytes) and its
//    output columns past N are never stored.
//  * Workgroups are renumbered so that the tiles sharing operand panels run
//    on one XCD and reuse them from that XCD's L2.  Where it fits the L2,
//    the skinny kernels instead put every split of a tile on one XCD, so
//    that the slab sum can read the slabs from the L2 that holds them.
//  * Slabs too large for the memory-side cache are stored as streaming
//    writes (stream_slabs).
//
// Which kernel and configuration serves a problem (the shape rules, the tile
// order, the persistent form) is decided in plan.cpp; this file holds the
// kernels, their launchers and the lists of instantiated configurations.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "splitk_internal.h"

namespace splitk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


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

// Output tile and split of skinny workgroup b (of n = tiles_m * tiles_n *
// splits).  Each XCD takes a contiguous range of logical ids.
//   order 0: row tile fastest, then column tile, then split: an XCD's
//            workgroups share the A and B panels of one split.
//   order 1: split fastest, then row tile, then column tile: every slab of a
//            tile is written on one XCD, and the slab sum that follows
//            (slab_reduce_tiles) visits the tiles in the same order, reading
//            the slabs from the L2 of the XCD that wrote them.  It costs the
//            GEMM the whole K range of fewer tiles per XCD, so the planner
//            takes it only where that still fits the XCD's L2.
struct TileId {
    int mt, nt, s;  // row tile, column tile, split
};
__device__ __attribute__((always_inline)) inline TileId skinny_tile(int b, int n, const TileGrid& g) {
    const uint32_t logical = (uint32_t)xcd_logical_id(b, n);
    if (g.order == 1) {
        const uint32_t u = fastdiv(logical, g.by_splits);
        const uint32_t nt = fastdiv(u, g.by_tiles_m);
        return TileId{(int)(u - nt * g.tiles_m), (int)nt, (int)(logical - u * g.splits)};
    }
    const uint32_t rest = fastdiv(logical, g.by_tiles_m);
    const uint32_t s = fastdiv(rest, g.by_tiles_n);
    return TileId{(int)(logical - rest * g.tiles_m), (int)(rest - s * g.tiles_n), (int)s};
}

// Calls f(integral_constant<int, I>) for I = B .. E-1: a loop whose index
// is a constant expression in the body.
template <int B, int E, class F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// LDS slot of 16-byte piece p of staged row r.  XOR-swizzled so that the
// fragment reads below (32 rows, one piece each) are conflict-free whether
// the LDS serves 8 or 16 lanes of a 16-byte read per cycle: over any 16
// consecutive rows, rows of equal parity get 8 distinct slots, and over any 8
// consecutive rows all slots differ.
__device__ inline int slot_of(int r, int p) { return p ^ (r & 7) ^ ((r >> 3) & 1); }

// ---------------------------------------------------------------------------
// B stored as [K,N] (n contiguous) instead of [N,K].
//
// A chunk of B is then CK k-rows of the tile's BN columns: CK*BN*ES bytes,
// the same 128 bytes per column as in the [N,K] case, held in LDS as the
// dense [CK][BN] tile.  Within each k-row the 16-byte granules are permuted
// (granule g sits at g ^ kn_flip(k-row)) so that the transposing fragment
// reads below, which take 4 consecutive k-rows x 64 bytes at once, meet 16
// distinct granule positions modulo the 256 bytes of the LDS banks.
// Granule positions modulo 16 of k-row r start at r * (granules per row):
// rows of 64 bytes already land in distinct quarters, rows of 128 bytes
// alternate halves and need the 64-byte block flipped on every other pair,
// and rows of 256 bytes or more all start at 0 and take the block index
// XOR r % 4.  The permutation stays inside a row, so each DMA instruction
// still fetches whole row segments.
template <int ES, int BN>
__device__ inline int kn_flip(int krow) {
    constexpr int RG = BN * ES / 16;  // granules per k-row
    return RG >= 16 ? 4 * (krow & 3) : (RG == 8 ? 4 * ((krow >> 1) & 1) : 0);
}

// LDS byte offset, inside the B tile, of byte colb of k-row krow.
template <int ES, int BN>
__device__ inline int kn_lds(int krow, int colb) {
    return krow * BN * ES + (((colb >> 4) ^ kn_flip<ES, BN>(krow)) << 4) + (colb & 15);
}

// Global byte offset, from the split's first k-row, of the 16 bytes that
// fill slot j of 128-byte unit u of the tile (the tile is filled unit by
// unit in LDS order) for the column tile starting at byte col0.  A tail
// tile's granules past the last column re-read the row's last granule (in
// bounds; those columns are never stored).  Needs row_bytes_b % 16 == 0.
template <int ES, int BN>
__device__ inline size_t kn_src(int u, int j, size_t row_bytes_b, size_t col0) {
    constexpr int RG = BN * ES / 16;
    const int pg = u * 8 + j;  // granule position in the tile
    const int krow = pg / RG;
    size_t col = col0 + (size_t)(((pg % RG) ^ kn_flip<ES, BN>(krow)) * 16);
    if (col + 16 > row_bytes_b) col = row_bytes_b - 16;
    return (size_t)krow * row_bytes_b + col;
}

// Cross-wave sum of a skinny workgroup's W partial BM x BN tiles, and its
// store.  Each wave writes its accumulators column-major into its own LDS
// tile (wave w's tile starts TS floats after wave w-1's): the four
// registers 4g..4g+3 of a 32x32 block hold four consecutive rows of one
// column, so each group is one 16-byte write.  A column pitch of BM + 4
// floats steps 16 bytes further round the banks per column, which keeps the
// lanes of a write (and of the reads below) on distinct banks.  Then each
// thread takes one column and four rows, adds the W tiles in ascending wave
// order and stores the four values.  Consecutive lanes hold consecutive
// columns, so every store instruction writes whole row segments; columns at
// or past `valid` (outside N) are not stored.  The caller guarantees that no
// other wave still reads a wave's tile area when that wave calls this: its
// own staging area (TS floats per wave, reused), or an area freed by a
// barrier.
template <int BM, int BN, int W, int MB, int NB, int TS>
__device__ inline void sum_and_store(float* lds, const f32x16 (&acc)[MB][NB], float* out, int N,
                                     int valid, int wave, int lane) {
    constexpr int CP = BM + 4;  // floats per column of one wave's tile
    static_assert(TS >= BN * CP, "tile stride");
    float* mine = lds + wave * TS;
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 v = {acc[mb][nb][4 * g], acc[mb][nb][4 * g + 1], acc[mb][nb][4 * g + 2],
                                 acc[mb][nb][4 * g + 3]};
                *(f32x4*)(mine + (nb * 32 + r) * CP + mb * 32 + 8 * g + 4 * h) = v;
            }
    // The slab pointer is needed only for the stores below; materialized
    // here, its argument load is not left on the path after the barrier.
    asm volatile("" ::"s"(out));
    __syncthreads();
    for (int it = threadIdx.x; it < BN * (BM / 4); it += W * 64) {
        const int col = it % BN, rq = it / BN;
        // All W reads first, then the adds in ascending wave order.
        f32x4 t[W];
#pragma unroll
        for (int w = 0; w < W; ++w) t[w] = *(const f32x4*)(lds + w * TS + col * CP + 4 * rq);
        __builtin_amdgcn_sched_group_barrier(0x100, W, 0);  // the reads ahead of every add
        f32x4 v = t[0];
#pragma unroll
        for (int w = 1; w < W; ++w) v += t[w];
        if (col < valid) {
            float* o = out + (size_t)(4 * rq) * N + col;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[(size_t)e * N] = v[e];
        }
    }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// MFMA B fragment of step q for the 32 columns of block nb from a [K,N]
// tile.  16-bit types: lane l needs B[16q + 8(l/32) + t][32nb + l%32] for
// t = 0..7, the same k slots as the A fragment (piece 2q + l/32 of its row).
// ds_read_tr16_b64 hands lane i of each group of 16 lanes element i%4 of the
// 8 bytes addressed by lane 4j + i/4 of the group, as its element j.  So a
// lane addresses 4 consecutive columns of one k-row: group g covers columns
// 16(g%2) .. +15 for k-rows 16q + 8(g/2) + j (j = 0..3), and a second read
// 4 k-rows further down gives t = 4..7.
template <int DT, int BN>
__device__ inline u32x4 kn_frag(const uint8_t* tile, int q, int nb, int lane) {
    if constexpr (DT == 0) {
        // F32: lane l needs B[8q + 4(l/32) + e][32nb + l%32] for e = 0..3.
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int krow = 8 * q + 4 * (lane >> 5) + e;
            v[e] = *(const uint32_t*)(tile + kn_lds<4, BN>(krow, (nb * 32 + (lane & 31)) * 4));
        }
        return v;
    } else {
        const int g = lane >> 4;
        const int krow = 16 * q + 8 * (g >> 1) + ((lane >> 2) & 3);
        const int colb = (nb * 32 + 16 * (g & 1) + 4 * (lane & 3)) * 2;
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + kn_lds<2, BN>(krow, colb)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + kn_lds<2, BN>(krow + 4, colb)));
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2.x, l2.y, h2.x, h2.y};
    }
}

// Skinny kernel: one BM x BN output tile of one split per workgroup.  Its W
// waves take the split's chunks round-robin (chunk c goes to wave c % W);
// each wave loads its chunks with coalesced 16-byte loads into registers, D
// chunks ahead, stages each in its own LDS area and reads MFMA fragments
// back, so waves never wait for one another until the cross-wave sum.  BL
// selects the layout of B ([N,K] or [K,N]).
template <int DT, int BM, int BN, int W, int D, int BL>
__global__ __launch_bounds__(W * 64) void gemm_bt_wavek(const uint8_t* __restrict__ A,
                                                        const uint8_t* __restrict__ B,
                                                        float* __restrict__ P, int M, int N, int K,
                                                        int kps, TileGrid tg) {
    using Op = Mfma<DT>;
    constexpr int ES = Op::kElemBytes;
    constexpr int CK = kChunkBytes / ES;  // elements per chunk
    constexpr int MB = BM / 32, NB = BN / 32;
    constexpr int ROWS = BM + BN;         // staged rows per chunk: A rows, then B rows
    constexpr int LOADS = ROWS / 8;       // 16-byte loads per lane per chunk
    static_assert(ROWS % 8 == 0, "tile rows");
    // One LDS block: per-wave staging buffers during the k loop, then (after
    // a barrier) the W partial tiles of the cross-wave sum.
    constexpr int STAGE_BYTES = W * ROWS * kChunkBytes;
    // Each wave's partial tile goes into its own staging area when it fits
    // there (no barrier needed first); otherwise all tiles go at the front
    // once every wave is done staging.
    constexpr bool OWN = BN * (BM + 4) * 4 <= ROWS * kChunkBytes;
    constexpr int RED_BYTES = W * BN * (BM + 4) * 4;  // sum_and_store's tiles
    __shared__ __attribute__((aligned(16))) uint8_t smem[STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES];

    const TileId tile = skinny_tile(blockIdx.x, gridDim.x, tg);
    const int mt = tile.mt, nt = tile.nt, s = tile.s;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 31;
    const int h = lane >> 5;

    const int k0 = s * kps;
    const int k1 = min(k0 + kps, K);
    const int nchunks = (k1 - k0 + CK - 1) / CK;
    // This wave owns chunks wave, wave + W, wave + 2W, ... (wave-uniform count).
    const int mine = wave < nchunks ? (nchunks - wave + W - 1) / W : 0;

    // Coalesced loads: load i of a lane covers staged row 8*i + lane/8 and
    // writes LDS slot lane%8 of it, so each load instruction of the wave reads
    // eight whole 128-byte row segments and writes 1 KiB of LDS contiguously.
    const size_t row_bytes = (size_t)K * ES;
    const size_t row_bytes_b = (size_t)N * ES;  // [K,N] layout: one k-row of B
    const int lrow = lane >> 3, lslot = lane & 7;
    // Row 8*i + lrow of the A (then B) rows: one base per operand and a
    // uniform stride of 8 rows, so that the loads go out without a 64-bit
    // multiply each.  B rows past N (a tail tile) re-read row N-1 (row
    // offsets grow with the row, so clamping the offset clamps the row);
    // those columns are never stored.  Every address stays B or A plus an
    // offset, so the compiler keeps global (not flat) loads.
    const size_t stride8 = (size_t)8 * row_bytes;
    const uint8_t* a0 = A + ((size_t)mt * BM + lrow) * row_bytes + (size_t)k0 * ES;
    const size_t b0 = ((size_t)nt * BN + lrow) * row_bytes + (size_t)k0 * ES;  // offsets from B
    const size_t b_last = (size_t)(N - 1) * row_bytes + (size_t)k0 * ES;
    const uint8_t* src[LOADS];
    int piece[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int row = 8 * i + lrow;
        piece[i] = slot_of(row, lslot);  // the global piece that lands in slot lslot
        if (BL == 1 && i >= BM / 8) {
            // Unit row - BM of the [CK][BN] tile; its slot lslot.
            src[i] = B + (size_t)k0 * row_bytes_b +
                     kn_src<ES, BN>(row - BM, lslot, row_bytes_b, (size_t)nt * BN * ES);
            piece[i] = 0;
        } else if (i < BM / 8) {
            src[i] = a0 + (size_t)i * stride8;
        } else {
            const size_t o = b0 + (size_t)(i - BM / 8) * stride8;
            src[i] = B + (o < b_last ? o : b_last);
        }
    }
    uint8_t* lds = smem + wave * ROWS * kChunkBytes;

    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};

    u32x4 stg[D][LOADS];

    // Chunk id of this wave's t-th chunk, clamped into range so that every
    // global load is unconditional (a clamped load re-reads a real chunk and
    // is never consumed).  Straight-line loads let the compiler wait for
    // exactly the stage it is about to use while later stages stay in flight.
    auto chunk_of = [&](int t) { return mine > 0 ? wave + min(t, mine - 1) * W : 0; };
    // The upper half of a chunk (pieces 4..7) lies past the slice end only in
    // the last chunk of a 16-bit slice whose length is an odd multiple of 32.
    auto half_chunk = [&](int c) { return k0 + c * CK + CK / 2 >= k1; };

    auto load = [&](int c, u32x4 (&t)[LOADS]) {
        // In a half chunk the lanes meant for pieces 4..7 re-read pieces 0..3
        // (in bounds); those slots are never consumed.  With B as [K,N] the
        // units holding k-rows CK/2.. re-read the rows CK/2 above instead.
        const bool half = half_chunk(c);
        const int mask = half ? 3 : 7;
        const size_t off = (size_t)c * kChunkBytes;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            if (BL == 1 && i >= BM / 8) {
                const size_t up = (half && i >= (BM + BN / 2) / 8) ? (size_t)(CK / 2) * row_bytes_b : 0;
                t[i] = *(const u32x4*)(src[i] + (size_t)c * CK * row_bytes_b - up);
            } else {
                t[i] = *(const u32x4*)(src[i] + off + (piece[i] & mask) * 16);
            }
        }
    };
    auto compute = [&](int c, u32x4 (&t)[LOADS]) {
        // Stage the chunk in this wave's LDS buffer (row 8*i + lane/8, slot lane%8).
#pragma unroll
        for (int i = 0; i < LOADS; ++i) *(u32x4*)(lds + i * 1024 + lane * 16) = t[i];
        // MFMA step q takes pieces 2q (lanes 0-31) and 2q+1 (lanes 32-63) of
        // each of the 32 rows of a block: 16 consecutive k for both operands.
        const int steps = half_chunk(c) ? 2 : 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q >= steps) break;
            u32x4 fa[MB], fb[NB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = mb * 32 + r;
                fa[mb] = *(const u32x4*)(lds + row * kChunkBytes + slot_of(row, 2 * q + h) * 16);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if (BL == 1) {
                    fb[nb] = kn_frag<DT, BN>(lds + BM * kChunkBytes, q, nb, lane);
                } else {
                    const int row = BM + nb * 32 + r;
                    fb[nb] = *(const u32x4*)(lds + row * kChunkBytes + slot_of(row, 2 * q + h) * 16);
                }
            }
#pragma unroll
            for (int e = 0; e < Op::kStepsPerPiece; ++e)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[mb][nb] = Op::step(fa[mb], fb[nb], acc[mb][nb], e);
        }
    };

    // Prologue: D chunks in flight before the first MFMA.
#pragma unroll
    for (int j = 0; j < D; ++j) load(chunk_of(j), stg[j]);
    // Steady state: consume stage j, then refill it with the chunk D ahead.
    int t = 0;
    for (; t + D < mine; t += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            compute(chunk_of(t + j), stg[j]);
            load(chunk_of(t + j + D), stg[j]);
        }
    }
    // Epilogue: the stages still holding real chunks (no loads issued here).
#pragma unroll
    for (int j = 0; j < D; ++j)
        if (t + j < mine) compute(chunk_of(t + j), stg[j]);

    if constexpr (!OWN) __syncthreads();  // every wave is done with its staging buffer
    sum_and_store<BM, BN, W, MB, NB, OWN ? ROWS * kChunkBytes / 4 : BN * (BM + 4)>(
        reinterpret_cast<float*>(smem), acc,
                                     P + ((size_t)s * M + (size_t)mt * BM) * N + (size_t)nt * BN, N,
                                     min(BN, N - nt * BN), wave, lane);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (gfx9 encoding; the LDS and export counters
// are left at their maxima, i.e. not waited on).
#define SPLITK_VMCNT(n) ((((n) & 0xF) | ((((n) >> 4) & 3) << 14)) | 0x70 | 0xF00)

// Workgroup barrier without the memory fence __syncthreads() adds (the
// fence would wait for every load in flight, including the prefetches this
// pipeline keeps in flight across barriers).  Each wave first waits for its
// own LDS reads, so no read of a buffer is outstanding when another wave is
// allowed to overwrite it; the "memory" clobber keeps the compiler from
// moving LDS accesses across it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Large-tile kernel: each workgroup owns a BM x BN output tile of one split
// and its WM x WN waves share every staged chunk.  Chunks (128 bytes of each
// of the BM + BN rows) travel from global memory straight into a ring of
// NBUF LDS buffers (global_load_lds_dwordx4: no register staging and no
// ds_write), NBUF - 1 chunks ahead of the one being multiplied.  One DMA
// instruction of a wave fills eight whole 128-byte row segments, i.e. 1 KiB
// of the buffer; the swizzle is applied on the global side (the lane that
// fills slot j of row r fetches piece slot_of(r, j)).  Accumulators are
// stored straight to the partial slab: for each accumulator register the 32
// lanes of a half-wave write 32 consecutive floats of one row.
template <int DT, int BM, int BN, int WM, int WN, int NBUF, int BL>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bt_tiled(const uint8_t* __restrict__ A,
                                                              const uint8_t* __restrict__ B,
                                                              float* __restrict__ P, int M, int N,
                                                              int K, int kps, int tiles_m,
                                                              int tiles_n, int streaming,
                                                              int stagger, int order) {
    using Op = Mfma<DT>;
    constexpr int ES = Op::kElemBytes;
    constexpr int CK = kChunkBytes / ES;
    constexpr int NW = WM * WN;               // waves
    constexpr int ROWS = BM + BN;             // staged rows per chunk
    constexpr int BUF = ROWS * kChunkBytes;   // bytes per LDS buffer
    constexpr int DPW = ROWS / 8 / NW;        // DMA instructions per wave per chunk
    constexpr int TM = BM / WM, TN = BN / WN; // per-wave sub-tile
    constexpr int MB = TM / 32, NB = TN / 32;
    constexpr int GM = 4;                     // row tiles per group of the tile order
    static_assert(ROWS % (8 * NW) == 0 && BM % 8 == 0, "staging split");
    static_assert((NBUF - 2) * DPW < 64, "vmcnt range");
    // DMA instruction i fills rows 8*(i*NW + wave) ..: for these sizes the
    // A rows, the B rows and (for B as [K,N]) the B units holding the second
    // half of a chunk's k-rows begin at the same i in every wave.
    constexpr int IA = BM / 8 / NW, IH = (BM + BN / 2) / 8 / NW;
    static_assert((BM / 8) % NW == 0 && ((BM + BN / 2) / 8) % NW == 0, "row split per wave");
    __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * BUF];

    // Tile order 0: split major; inside a split, groups of GM row tiles
    // sweep all column tiles, so the workgroups resident on one XCD at a time
    // share a few A and B panels in its L2.  Order 1: split fastest, then M,
    // then N, so that every slab of a tile comes from one XCD (each XCD
    // takes a contiguous range of logical ids) and the tile-ordered slab sum
    // finds it in that XCD's L2.
    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    const int per_split = tiles_m * tiles_n;
    int s, mt, nt;
    if (order == 1) {
        const int splits = gridDim.x / per_split;
        const int t = logical / splits;
        s = logical - t * splits;
        nt = t / tiles_m;
        mt = t - nt * tiles_m;
    } else {
        s = logical / per_split;
        const int t = logical % per_split;
        const int gm = min(GM, tiles_m);
        const int group = t / (gm * tiles_n);
        const int in_group = t % (gm * tiles_n);
        const int rows_here = min(gm, tiles_m - group * gm);
        mt = group * gm + in_group % rows_here;
        nt = in_group / rows_here;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // Uniform in a wave; as a scalar it gives the DMA instructions' LDS
    // addresses without a lane read per instruction.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int r = lane & 31;
    const int h = lane >> 5;

    const int k0 = s * kps;
    const int k1 = min(k0 + kps, K);
    const int nchunks = (k1 - k0 + CK - 1) / CK;
    auto half_chunk = [&](int c) { return k0 + c * CK + CK / 2 >= k1; };

    // DMA instruction i of this wave fills rows 8*g .. 8*g+7 (g = i*NW + wave)
    // of a buffer; this lane fills slot lane%8 of row 8*g + lane/8.
    const size_t row_bytes = (size_t)K * ES;
    const size_t row_bytes_b = (size_t)N * ES;  // [K,N] layout: one k-row of B
    const uint8_t* src[DPW];
    int piece[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
        const int row = 8 * (i * NW + wave) + (lane >> 3);
        piece[i] = slot_of(row, lane & 7);
        if (BL == 1 && i >= IA) {
            src[i] = B + (size_t)k0 * row_bytes_b +
                     kn_src<ES, BN>(row - BM, lane & 7, row_bytes_b, (size_t)nt * BN * ES);
            piece[i] = 0;
        } else {
            src[i] = (row < BM ? A + (size_t)(mt * BM + row) * row_bytes
                               : B + (size_t)min(nt * BN + row - BM, N - 1) * row_bytes) +
                     (size_t)k0 * ES;
        }
    }
    // Chunk 0 address of each DMA instruction for a full chunk, the piece
    // folded in: a full chunk c adds one uniform offset.
    const uint8_t* full[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) full[i] = src[i] + piece[i] * 16;
    // In a half chunk the lanes meant for pieces 4..7 re-read pieces 0..3
    // (in bounds); those copies are finite and meet zero A fragments in
    // compute().  That is piece & 3 instead of piece, i.e. (piece & 4) * 16
    // bytes lower.  Bit 2 of a lane's piece is the same in every instruction:
    // slot_of(8g + lane/8, lane%8) differs between row groups g only in bit 0.
    const int half_back = (slot_of(lane >> 3, lane & 7) & 4) * 16;
    // DMA instructions [lo, hi) of chunk c, into ring slot c % NBUF.
    // `may_be_half` false: the caller knows chunk c is full.
    auto dma = [&](int c, int lo, int hi, auto may_be_half) {
        uint8_t* buf = smem + (c % NBUF) * BUF;
        const bool half = decltype(may_be_half)::value && half_chunk(c);
        const size_t off = (size_t)c * kChunkBytes;
        const size_t off_kn = (size_t)c * CK * row_bytes_b;
#pragma unroll
        for (int i = lo; i < hi; ++i) {
            const uint8_t* g;
            if (BL == 1 && i >= IA) {
                // B as [K,N]: in a half chunk the second half of the k-rows
                // re-reads the first half (in bounds, never consumed).
                g = full[i] + off_kn - ((half && i >= IH) ? (size_t)(CK / 2) * row_bytes_b : 0);
            } else {
                g = full[i] + off - (half ? half_back : 0);
            }
            __builtin_amdgcn_global_load_lds((const void*)g,
                                             (__attribute__((address_space(3))) void*)(buf + (i * NW + wave) * 1024),
                                             16, 0, 0);
        }
    };

    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};

    // MFMA work of chunk c.  When `next` >= 0 the DMA of chunk `next` is
    // issued between this chunk's MFMAs.  Issued all at once, the wave
    // stalled ~1200 cycles per chunk waiting for the texture path to accept
    // it, with no MFMA in flight (256x256 tiles: spread, the chunk's work
    // went from ~4100 to ~3550 cycles).
    //  * Two-buffer ring (256x256 tiles): the next chunk is the only one in
    //    flight, so it is issued over the first two of the four k-steps, one
    //    instruction per MFMA pair, pinned with scheduling barriers (the
    //    scheduler otherwise bunches them).  Issued over all four k-steps,
    //    its last quarter had no time to land before it was needed.
    //  * Deeper rings: a quarter after each k-step, as the scheduler places it.
    constexpr int DMA_STEPS = NBUF == 2 ? 2 : 4;
    // `may_be_half` is false for the steady-state chunks: only a split's last
    // chunk can be half empty, and it always falls in the tail loop.
    auto compute = [&](int c, int next, auto may_be_half, auto next_may_be_half) {
        const uint8_t* lds = smem + (c % NBUF) * BUF;
        const int steps = (decltype(may_be_half)::value && half_chunk(c)) ? 2 : 4;
        // Fragments of k-step q into fa[q % 2], fb[q % 2].  With the
        // two-buffer ring (PIPE) step q + 1's are read while step q's MFMAs
        // run, pinned by scheduling groups: 1-2% on 256x256 tiles.  The
        // deeper rings keep the compiler's order, reads just before their
        // step (the pinned order was 6% slower on 256x128 with 2x4 waves).
        constexpr bool PIPE = NBUF == 2;
        u32x4 fa[2][MB], fb[2][NB];
        auto frags = [&](auto qv) {
            constexpr int q = decltype(qv)::value;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = wm * TM + mb * 32 + r;
                u32x4 v = *(const u32x4*)(lds + row * kChunkBytes + slot_of(row, 2 * q + h) * 16);
                if (decltype(may_be_half)::value && q >= 2) v = q < steps ? v : u32x4{};
                fa[q & 1][mb] = v;
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if (BL == 1) {
                    fb[q & 1][nb] = kn_frag<DT, BN>(lds + BM * kChunkBytes, q, wn * (TN / 32) + nb, lane);
                } else {
                    const int row = BM + wn * TN + nb * 32 + r;
                    fb[q & 1][nb] = *(const u32x4*)(lds + row * kChunkBytes + slot_of(row, 2 * q + h) * 16);
                }
            }
        };
        constexpr int NREAD = MB + NB * (BL == 1 ? (DT == 0 ? 4 : 2) : 1);  // LDS reads per step
        constexpr int NM = Op::kStepsPerPiece * MB * NB;                     // MFMAs per step
        frags(std::integral_constant<int, 0>{});
        if constexpr (PIPE) __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);  // step 0's reads first
        static_for<0, 4>([&](auto qv) {
            constexpr int q = decltype(qv)::value;
            if constexpr (PIPE && q < 3) frags(std::integral_constant<int, q + 1>{});
            if constexpr (!PIPE && q > 0) frags(qv);
#pragma unroll
            for (int e = 0; e < Op::kStepsPerPiece; ++e)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[mb][nb] = Op::step(fa[q & 1][mb], fb[q & 1][nb], acc[mb][nb], e);
            // Schedule: the next step's LDS reads ahead of this step's MFMAs.
            if constexpr (PIPE && q < 3) __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
            bool pinned = !PIPE;
            if constexpr (q < DMA_STEPS) {
                constexpr int LO = q * DPW / DMA_STEPS, ND = (q + 1) * DPW / DMA_STEPS - LO;
                if (next >= 0) {
                    dma(next, LO, LO + ND, next_may_be_half);
                    if constexpr (NBUF == 2) {
                        static_for<0, ND>([&](auto jv) {
                            constexpr int j = decltype(jv)::value;
                            constexpr int G = (j + 1) * NM / ND - j * NM / ND;  // MFMAs before DMA j
                            if constexpr (G > 0) __builtin_amdgcn_sched_group_barrier(0x008, G, 0);
                            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one VMEM load
                        });
                        pinned = true;
                    }
                }
            }
            if (!pinned) __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
        });
    };

    // Prologue: the first NBUF - 1 chunks in flight.
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j)
        if (j < nchunks) dma(j, 0, DPW, std::true_type{});
    // Staggered start.  On a grid of several rounds the CUs would otherwise
    // run in lockstep: all of them store their partial tiles at the same
    // moment, each at 1/256 of the write bandwidth while no MFMA work runs
    // anywhere.  The first round's workgroups (one per CU) wait 512 cycles
    // per slot of their XCD, 0 to 31 slots, once their first chunks are in
    // flight, which spreads the store phases over about one tile's store time.
    if ((int)blockIdx.x < stagger) {
        const int slot = (blockIdx.x >> 3) & 31;
        for (int i = 0; i < slot; ++i) __builtin_amdgcn_s_sleep(8);
    }
    // Steady state: every pass issues one more chunk, so exactly NBUF - 2
    // younger chunks (DPW loads each) are outstanding behind chunk c.  Only
    // a split's last chunk can be half empty: the passes before the one
    // that issues it know that both their chunk and the issued one are full.
    int c = 0;
    for (; c + NBUF < nchunks; ++c) {
        __builtin_amdgcn_s_waitcnt(SPLITK_VMCNT((NBUF - 2) * DPW));
        lds_barrier();  // chunk c complete for all waves; slot of chunk c-1 free
        compute(c, c + NBUF - 1, std::false_type{}, std::false_type{});
    }
    if (c + NBUF - 1 < nchunks) {  // issues the last chunk
        __builtin_amdgcn_s_waitcnt(SPLITK_VMCNT((NBUF - 2) * DPW));
        lds_barrier();
        compute(c, c + NBUF - 1, std::false_type{}, std::true_type{});
        ++c;
    }
    // Tail: no more loads to issue; wait for everything still in flight.
    for (; c < nchunks; ++c) {
        __builtin_amdgcn_s_waitcnt(SPLITK_VMCNT(0));
        lds_barrier();
        compute(c, -1, std::true_type{}, std::true_type{});
    }

    // Register i of lane l holds row 8*(i/4) + 4*(l/32) + i%4, column l%32.
    // The lane's own part (row 4*(l/32), column l%32) goes into one base
    // pointer; the rest of each row offset is the same for the whole wave.
    float* base = P + ((size_t)s * M + (size_t)mt * BM + wm * TM + 4 * h) * N + (size_t)nt * BN +
                  wn * TN + r;
    const int valid = N - (nt * BN + wn * TN);  // columns of this wave's sub-tile inside N
    // Slabs too large for the memory-side cache (stream_slabs) are stored
    // as streaming (nontemporal) writes: they are read once, by the slab
    // sum, and so do not displace the operands.
    if (valid >= TN && streaming) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float* row = base + (size_t)(mb * 32 + 8 * (i >> 2) + (i & 3)) * (size_t)N;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) __builtin_nontemporal_store(acc[mb][nb][i], &row[nb * 32]);
            }
    } else if (valid >= TN) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float* row = base + (size_t)(mb * 32 + 8 * (i >> 2) + (i & 3)) * (size_t)N;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) row[nb * 32] = acc[mb][nb][i];
            }
    } else {
        // Tail tile: only the columns inside N.
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float* row = base + (size_t)(mb * 32 + 8 * (i >> 2) + (i & 3)) * (size_t)N;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    if (nb * 32 + r < valid) row[nb * 32] = acc[mb][nb][i];
            }
    }
}

template <int DT, int BM, int BN, int WM, int WN, int NBUF, int BL>
hipError_t launch_tiled(const void* A, const void* B, float* P, int64_t M, int64_t N, int64_t K,
                        int64_t kps, int64_t splits, int order, hipStream_t stream) {
    const int tiles_m = (int)(M / BM), tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * (int64_t)tiles_n * splits));
    const dim3 block(WM * WN * 64);
    const uint8_t* a = (const uint8_t*)A;
    const uint8_t* b = (const uint8_t*)B;
    int m = (int)M, n = (int)N, k = (int)K, kp = (int)kps;
    int streaming = stream_slabs(splits, M, N) ? 1 : 0;
    // Every instantiated tile needs a whole CU (LDS ring of 128-144 KiB), so
    // the first device_cus() workgroups are the first round.
    const int cus = device_cus();
    int stagger = (int64_t)grid.x > cus ? cus : 0;
    void* args[] = {&a, &b, &P, &m, &n, &k, &kp, (void*)&tiles_m, (void*)&tiles_n, &streaming, &stagger,
                    &order};
    return hipLaunchKernel((const void*)&gemm_bt_tiled<DT, BM, BN, WM, WN, NBUF, BL>, grid, block, args,
                           0, stream);
}

// Sixteen zero bytes: the A pieces of the empty upper half of a half chunk
// are loaded from here by the persistent large-tile kernel.
__device__ __attribute__((aligned(64))) uint32_t kZeroPiece[4];

// Persistent form of the large-tile kernel for grids of several rounds (two-
// buffer ring; B as [N,K], or as [K,N] with BL = 1, staged and read as in
// the one-tile kernel).  One workgroup per CU walks a sequence of tiles
// instead of ending after one, and its LDS ring runs on across tiles: the
// next tile's first chunk is loaded while this tile's last chunk is
// multiplied, and lands while this tile's partials are being stored.  A
// wave's vector-memory operations complete in the order it issued them
// (loads into LDS and stores alike), so once 64 or more store instructions
// have been issued after that load, a counter of at most 63 outstanding
// operations means that it has landed: the next tile starts multiplying
// while the last of its stores drain, where the one-tile kernel pays a
// workgroup's start and its first chunk's full latency once per tile.
// (Loading the second chunk before the stores as well, into the slot the
// last chunk frees, was 2-4% slower: that pass then had nothing to load.)
//
// Tile sequence: the tiles are numbered as in the one-tile kernel (split
// major; groups of GM row tiles sweep the column tiles) and each XCD takes a
// contiguous range of them.  Workgroup b runs on XCD x = b % 8 as its
// (b / 8)-th workgroup there; of the wg_x workgroups on XCD x, workgroup j
// takes tiles j, j + wg_x, j + 2 wg_x, ... of that range.  This is a
// bijection onto all tiles as long as every XCD has a workgroup (gridDim.x
// >= 8) and no XCD has more workgroups than tiles (gridDim.x <= tiles).
template <int DT, int BM, int BN, int WM, int WN, int BL>
__global__ __launch_bounds__(WM * WN * 64) void gemm_bt_tiled_pt(const uint8_t* __restrict__ A,
                                                                 const uint8_t* __restrict__ B,
                                                                 float* __restrict__ P, int M, int N,
                                                                 int K, int kps, int tiles_m,
                                                                 int tiles_n, int splits,
                                                                 int streaming, int stagger) {
    using Op = Mfma<DT>;
    constexpr int NBUF = 2;
    constexpr int ES = Op::kElemBytes;
    constexpr int CK = kChunkBytes / ES;
    constexpr int NW = WM * WN;
    constexpr int ROWS = BM + BN;
    constexpr int BUF = ROWS * kChunkBytes;
    constexpr int DPW = ROWS / 8 / NW;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MB = TM / 32, NB = TN / 32;
    constexpr int GM = 4;
    // [K,N]: DMA instructions [IA, DPW) fill the B part, [IH, DPW) its second
    // half of the k-rows.
    constexpr int IA = BM / 8 / NW, IH = (BM + BN / 2) / 8 / NW;
    // A whole sub-tile's partial store is MB * 16 * NB store instructions per
    // wave; the wait at the start of the next tile counts on at least 64.
    static_assert(MB * 16 * NB >= 64, "tile too small for the cross-tile wait");
    static_assert(ROWS % (8 * NW) == 0 && BM % 8 == 0, "staging split");
    // The ring, then 1 KiB per wave that dummy loads write into.
    __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * BUF + NW * 1024];

    const int per_split = tiles_m * tiles_n;
    const int total = per_split * splits;
    const int x = blockIdx.x & 7, j8 = blockIdx.x >> 3;
    const int q8 = total >> 3, r8 = total & 7;
    const int start_x = x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8;
    const int count_x = q8 + (x < r8 ? 1 : 0);
    const int wg_x = ((int)gridDim.x >> 3) + (x < ((int)gridDim.x & 7) ? 1 : 0);
    const int gm = min(GM, tiles_m);
    auto decode = [&](int local, int& s, int& mt, int& nt) __attribute__((always_inline)) {
        const int logical = start_x + local;
        s = logical / per_split;
        const int t = logical - s * per_split;
        const int group = t / (gm * tiles_n);
        const int in_group = t - group * (gm * tiles_n);
        const int rows_here = min(gm, tiles_m - group * gm);
        nt = in_group / rows_here;
        mt = group * gm + (in_group - nt * rows_here);
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int r = lane & 31;
    const int h = lane >> 5;
    const size_t row_bytes = (size_t)K * ES;
    const size_t row_bytes_b = (size_t)N * ES;  // [K,N] layout: one k-row of B

    // Chunk-0 address of each DMA instruction of this wave, piece folded in,
    // for the tile whose chunks are being loaded (the "load tile"), and that
    // tile's k range and chunk count.
    const uint8_t* full[DPW];
    int k0 = 0, k1 = 0, nch = 0;
    auto set_load_tile = [&](int s, int mt, int nt) __attribute__((always_inline)) {
        k0 = s * kps;
        k1 = min(k0 + kps, K);
        nch = (k1 - k0 + CK - 1) / CK;
#pragma unroll
        for (int i = 0; i < DPW; ++i) {
            const int row = 8 * (i * NW + wave) + (lane >> 3);
            if (BL == 1 && i >= IA) {
                full[i] = B + (size_t)k0 * row_bytes_b +
                          kn_src<ES, BN>(row - BM, lane & 7, row_bytes_b, (size_t)nt * BN * ES);
            } else {
                const uint8_t* src = (row < BM ? A + (size_t)(mt * BM + row) * row_bytes
                                               : B + (size_t)min(nt * BN + row - BM, N - 1) * row_bytes) +
                                     (size_t)k0 * ES;
                full[i] = src + slot_of(row, lane & 7) * 16;
            }
        }
    };
    // A half-empty chunk is always the load tile's last: before it is issued
    // the lanes meant for pieces 4..7 are redirected for good.  A rows read
    // the zero piece (their upper half of the chunk is zero, so the MFMAs
    // need no masking), B rows re-read pieces 0..3 (in bounds, finite).  Bit
    // 2 of a lane's piece is the same in every instruction: slot_of(8g +
    // lane/8, lane%8) differs between row groups g only in bit 0.
    const bool upper = (slot_of(lane >> 3, lane & 7) & 4) != 0;
    // With B as [K,N] the instructions of the second half of the k-rows
    // re-read the first half instead (in bounds, finite, and met by the zero
    // upper half of the A rows).
    auto make_half = [&](int c) __attribute__((always_inline)) {
        if (upper) {
#pragma unroll
            for (int i = 0; i < DPW; ++i) {
                if (8 * (i * NW + wave) < BM)
                    full[i] = (const uint8_t*)((uintptr_t)kZeroPiece - (uintptr_t)c * kChunkBytes);
                else if (BL == 0)
                    full[i] -= 64;
            }
        }
        if (BL == 1) {
#pragma unroll
            for (int i = IH; i < DPW; ++i) full[i] -= (size_t)(CK / 2) * row_bytes_b;
        }
    };
    // The DMA instructions [lo, hi) of chunk c of the load tile into ring
    // slot `slot`.  With c < 0 they are dummies: they re-read the load tile's
    // last issued chunk (chunk `last`, whose addresses are valid whatever
    // make_half did) into a spare LDS area that nothing reads.  The last
    // pass of the last tile, which has nothing to load, then still issues
    // the same instructions, so the MFMA sequence around them needs no
    // branch.
    auto dma = [&](int slot, int c, int last, int lo, int hi) __attribute__((always_inline)) {
        const bool dummy = c < 0;
        const int cc = dummy ? last : c;
        const size_t off = (size_t)cc * kChunkBytes;
        const size_t off_kn = (size_t)cc * CK * row_bytes_b;  // [K,N]: CK k-rows per chunk
        uint8_t* dst = dummy ? smem + NBUF * BUF + wave * 1024 : smem + slot * BUF + wave * 1024;
        const int step = dummy ? 0 : NW * 1024;
#pragma unroll
        for (int i = lo; i < hi; ++i) {
            const uint8_t* g = full[i] + ((BL == 1 && i >= IA) ? off_kn : off);
            __builtin_amdgcn_global_load_lds((const void*)g, (__attribute__((address_space(3))) void*)(dst + i * step),
                                             16, 0, 0);
        }
    };

    f32x16 acc[MB][NB];

    // MFMA work of the chunk in ring slot `slot`, with chunk next_c of the
    // load tile (or dummies, next_c < 0) issued into ring slot next_slot
    // between the MFMAs: one load per MFMA pair over the first two k-steps,
    // as in the one-tile kernel's two-buffer ring.
    auto compute = [&](int slot, int next_slot, int next_c, int last) __attribute__((always_inline)) {
        const uint8_t* lds = smem + slot * BUF;
        u32x4 fa[2][MB], fb[2][NB];
        auto frags = [&](auto qv) __attribute__((always_inline)) {
            constexpr int q = decltype(qv)::value;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = wm * TM + mb * 32 + r;
                fa[q & 1][mb] = *(const u32x4*)(lds + row * kChunkBytes + slot_of(row, 2 * q + h) * 16);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if (BL == 1) {
                    fb[q & 1][nb] = kn_frag<DT, BN>(lds + BM * kChunkBytes, q, wn * (TN / 32) + nb, lane);
                } else {
                    const int row = BM + wn * TN + nb * 32 + r;
                    fb[q & 1][nb] = *(const u32x4*)(lds + row * kChunkBytes + slot_of(row, 2 * q + h) * 16);
                }
            }
        };
        constexpr int NREAD = MB + NB * (BL == 1 ? (DT == 0 ? 4 : 2) : 1);  // LDS reads per step
        constexpr int NM = Op::kStepsPerPiece * MB * NB;
        constexpr int DMA_STEPS = 2;
        frags(std::integral_constant<int, 0>{});
        __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
        static_for<0, 4>([&](auto qv) {
            constexpr int q = decltype(qv)::value;
            if constexpr (q < 3) frags(std::integral_constant<int, q + 1>{});
#pragma unroll
            for (int e = 0; e < Op::kStepsPerPiece; ++e)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[mb][nb] = Op::step(fa[q & 1][mb], fb[q & 1][nb], acc[mb][nb], e);
            if constexpr (q < 3) __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
            if constexpr (q < DMA_STEPS) {
                constexpr int LO = q * DPW / DMA_STEPS, ND = (q + 1) * DPW / DMA_STEPS - LO;
                dma(next_slot, next_c, last, LO, LO + ND);
                static_for<0, ND>([&](auto jv) {
                    constexpr int j = decltype(jv)::value;
                    constexpr int G = (j + 1) * NM / ND - j * NM / ND;
                    if constexpr (G > 0) __builtin_amdgcn_sched_group_barrier(0x008, G, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                });
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
            }
        });
    };

    int local = j8;
    int s, mt, nt;
    decode(local, s, mt, nt);
    set_load_tile(s, mt, nt);
    if (k0 + CK / 2 >= k1) make_half(0);
    dma(0, 0, 0, 0, DPW);
    if ((int)blockIdx.x < stagger) {
        const int slot = (blockIdx.x >> 3) & 31;
        for (int i = 0; i < slot; ++i) __builtin_amdgcn_s_sleep(8);
    }
    int rb = 0;          // ring slot of this tile's chunk 0
    bool lead = false;   // this tile's chunk 0 was issued before the last tile's stores
    int issued = 0;      // last issued chunk of the load tile
    for (;;) {
        // The load tile is this tile until its last chunk is multiplied.
        const int cs = s, cmt = mt, cnt = nt, cn = nch;
        const int next_local = local + wg_x;
        const bool more = next_local < count_x;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};
        for (int c = 0; c < cn; ++c) {
            // Chunk c issues chunk c + 1, except that the last one issues the
            // next tile's chunk 0 (which then becomes the load tile), or
            // dummies in the last tile.
            int next_c = c + 1;
            if (c == cn - 1) {
                next_c = -1;
                if (more) {
                    decode(next_local, s, mt, nt);
                    set_load_tile(s, mt, nt);
                    next_c = 0;
                }
            }
            if (next_c >= 0) {
                if (next_c == nch - 1 && k0 + next_c * CK + CK / 2 >= k1) make_half(next_c);
                issued = next_c;
            }
            // At least 64 stores were issued after a lead tile's chunk 0: with
            // at most 63 operations outstanding, it has landed.  Chunk 1 went
            // out after the stores, so its wait covers them too.
            if (lead && c == 0)
                __builtin_amdgcn_s_waitcnt(SPLITK_VMCNT(63));
            else
                __builtin_amdgcn_s_waitcnt(SPLITK_VMCNT(0));
            lds_barrier();
            compute((rb + c) & 1, (rb + c + 1) & 1, next_c, issued);
        }

        float* base = P + ((size_t)cs * M + (size_t)cmt * BM + wm * TM + 4 * h) * N + (size_t)cnt * BN +
                      wn * TN + r;
        const int valid = N - (cnt * BN + wn * TN);
        if (valid >= TN && streaming) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float* row = base + (size_t)(mb * 32 + 8 * (i >> 2) + (i & 3)) * (size_t)N;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) __builtin_nontemporal_store(acc[mb][nb][i], &row[nb * 32]);
                }
        } else if (valid >= TN) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float* row = base + (size_t)(mb * 32 + 8 * (i >> 2) + (i & 3)) * (size_t)N;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) row[nb * 32] = acc[mb][nb][i];
                }
        } else {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float* row = base + (size_t)(mb * 32 + 8 * (i >> 2) + (i & 3)) * (size_t)N;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        if (nb * 32 + r < valid) row[nb * 32] = acc[mb][nb][i];
                }
            // Fewer store instructions may have been issued here: wait for
            // all of them, so the next tile's first wait holds.
            __builtin_amdgcn_s_waitcnt(SPLITK_VMCNT(0));
        }
        if (!more) {
            // The dummy loads of the last chunk must land before the
            // workgroup's LDS is released.
            __builtin_amdgcn_s_waitcnt(SPLITK_VMCNT(0));
            break;
        }
        rb = (rb + cn) & 1;
        local = next_local;
        lead = true;
    }
}

template <int DT, int BM, int BN, int WM, int WN, int BL>
hipError_t launch_tiled_pt(const void* A, const void* B, float* P, int64_t M, int64_t N, int64_t K,
                           int64_t kps, int64_t splits, hipStream_t stream) {
    const int tiles_m = (int)(M / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int64_t tiles = tiles_m * (int64_t)tiles_n * splits;
    const int64_t g = std::min<int64_t>(tiles, std::max(8, device_cus() & ~7));
    if (g < 8) return hipErrorInvalidConfiguration;  // every XCD needs a workgroup
    const dim3 grid((unsigned)g);
    const dim3 block(WM * WN * 64);
    const uint8_t* a = (const uint8_t*)A;
    const uint8_t* b = (const uint8_t*)B;
    int m = (int)M, n = (int)N, k = (int)K, kp = (int)kps, sp = (int)splits;
    int streaming = stream_slabs(splits, M, N) ? 1 : 0;
    int stagger = tiles > g ? (int)g : 0;
    void* args[] = {&a, &b, &P, &m, &n, &k, &kp, (void*)&tiles_m, (void*)&tiles_n, &sp, &streaming, &stagger};
    return hipLaunchKernel((const void*)&gemm_bt_tiled_pt<DT, BM, BN, WM, WN, BL>, grid, block, args, 0, stream);
}

// Instantiated shared-ring configurations: (BM, BN, WM, WN, NBUF), NBUF
// chunk buffers in the LDS ring (at most 160 KiB).
#define SPLITK_TILED_CONFIGS(X) \
    X(256, 256, 2, 2, 2)        \
    X(256, 128, 2, 2, 3)        \
    X(256, 128, 2, 4, 3)        \
    X(128, 128, 2, 2, 4)

// Instantiated persistent configurations (two-buffer ring): (BM, BN, WM, WN).
#define SPLITK_TILED_PT_CONFIGS(X) \
    X(256, 256, 2, 2)              \
    X(256, 128, 2, 2)              \
    X(256, 128, 2, 4)
#define SPLITK_KN_TILED_PT_CONFIGS(X) \
    X(256, 256, 2, 2)

// Skinny kernel with the last chunk by LDS DMA.  Same work split as
// gemm_bt_wavek (waves take a split's chunks round-robin, partial tiles
// summed through LDS), but each wave's last chunk travels from global memory
// straight into a private LDS area (global_load_lds_dwordx4), issued after
// the register loads of its earlier R chunks.  The last chunks are the ones
// every wave receives at the same moment; writing them to LDS with ds_write
// would queue eight waves' LDS writes at the very end.  Earlier chunks are
// transposed into fragments block by block (32 rows at a time) through a
// 4 KiB area, so one wave needs 4 KiB + one chunk of LDS.  A wave holds at
// most R + 1 chunks; the host only picks this kernel when that is enough.
template <int DT, int BM, int BN, int W, int R>
__global__ __launch_bounds__(W * 64) void gemm_bt_wavek_dma(const uint8_t* __restrict__ A,
                                                            const uint8_t* __restrict__ B,
                                                            float* __restrict__ P, int M, int N,
                                                            int K, int kps, TileGrid tg) {
    using Op = Mfma<DT>;
    constexpr int ES = Op::kElemBytes;
    constexpr int CK = kChunkBytes / ES;
    constexpr int MB = BM / 32, NB = BN / 32;
    constexpr int ROWS = BM + BN;
    constexpr int LOADS = ROWS / 8;
    constexpr int BLOCK = 32 * kChunkBytes;          // one 32-row block of a chunk
    static_assert(LOADS < 64 && R * LOADS + LOADS < 64, "vmcnt range");
    static_assert(BN * (BM + 4) * 4 <= ROWS * kChunkBytes, "a wave's reduction tile fits its DMA area");
    // Separate LDS objects for the transpose blocks and the DMA chunks, so
    // the compiler can see that writing a transpose block does not have to
    // wait for the DMA still in flight.  Each wave's reduction tile reuses
    // that wave's own DMA area.
    __shared__ __attribute__((aligned(16))) uint8_t tr_lds[W][BLOCK];
    __shared__ __attribute__((aligned(16))) uint8_t dma_lds[W][ROWS * kChunkBytes];

    const TileId tile = skinny_tile(blockIdx.x, gridDim.x, tg);
    const int mt = tile.mt, nt = tile.nt, s = tile.s;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 31;
    const int h = lane >> 5;

    const int k0 = s * kps;
    const int k1 = min(k0 + kps, K);
    const int nchunks = (k1 - k0 + CK - 1) / CK;
    const int mine = wave < nchunks ? (nchunks - wave + W - 1) / W : 0;
    // Chunk ids, clamped into range so that every load is unconditional; a
    // wave with fewer than R + 1 chunks re-reads real chunks it never uses.
    auto chunk_of = [&](int t) { return mine > 0 ? wave + min(max(t, 0), mine - 1) * W : 0; };
    auto half_chunk = [&](int c) { return k0 + c * CK + CK / 2 >= k1; };

    const size_t row_bytes = (size_t)K * ES;
    const int lrow = lane >> 3;
    // As in gemm_bt_wavek: per-operand bases, a uniform 8-row stride, B rows
    // past N clamped to row N-1 by their offset.
    const size_t stride8 = (size_t)8 * row_bytes;
    const uint8_t* a0 = A + ((size_t)mt * BM + lrow) * row_bytes + (size_t)k0 * ES;
    const size_t b0 = ((size_t)nt * BN + lrow) * row_bytes + (size_t)k0 * ES;  // offsets from B
    const size_t b_last = (size_t)(N - 1) * row_bytes + (size_t)k0 * ES;
    const uint8_t* src[LOADS];
    int piece[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        if (i < BM / 8) {
            src[i] = a0 + (size_t)i * stride8;
        } else {
            const size_t o = b0 + (size_t)(i - BM / 8) * stride8;
            src[i] = B + (o < b_last ? o : b_last);
        }
        piece[i] = slot_of(8 * i + lrow, lane & 7);
    }
    uint8_t* tr = &tr_lds[wave][0];            // 4 KiB transpose block
    uint8_t* dma_area = &dma_lds[wave][0];     // one whole chunk

    f32x16 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x16{};

    auto mfma_chunk = [&](const u32x4 (&fa)[MB][4], const u32x4 (&fb)[NB][4], int c) {
        const int steps = half_chunk(c) ? 2 : 4;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < Op::kStepsPerPiece; ++e)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const u32x4 a = q >= 2 && q >= steps ? u32x4{} : fa[mb][q];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = Op::step(a, fb[nb][q], acc[mb][nb], e);
                }
    };

    // Register chunks: loads issued first.
    u32x4 stg[R > 0 ? R : 1][LOADS];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int c = chunk_of(j);
        const size_t off = (size_t)c * kChunkBytes;
        const int mask = half_chunk(c) ? 3 : 7;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) stg[j][i] = *(const u32x4*)(src[i] + off + (piece[i] & mask) * 16);
    }
    // Last chunk: LDS DMA, issued after them (its rows 8i..8i+7 land at i KiB).
    {
        const int c = chunk_of(mine - 1);
        const size_t off = (size_t)c * kChunkBytes;
        const int mask = half_chunk(c) ? 3 : 7;
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(src[i] + off + (piece[i] & mask) * 16),
                                             (__attribute__((address_space(3))) void*)(dma_area + i * 1024),
                                             16, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    // Register chunks, oldest first: each 32-row block goes through the
    // transpose area (ds_write four loads, ds_read four fragments).
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j < mine - 1) {
            u32x4 fa[MB][4], fb[NB][4];
#pragma unroll
            for (int blk = 0; blk < MB + NB; ++blk) {
#pragma unroll
                for (int i = 0; i < 4; ++i) *(u32x4*)(tr + i * 1024 + lane * 16) = stg[j][blk * 4 + i];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4 v = *(const u32x4*)(tr + r * kChunkBytes + slot_of(r, 2 * q + h) * 16);
                    if (blk < MB) fa[blk][q] = v; else fb[blk - MB][q] = v;
                }
            }
            mfma_chunk(fa, fb, chunk_of(j));
        }
    }
    // The DMA chunk: wait for every load of this wave (it was issued last).
    __builtin_amdgcn_s_waitcnt(SPLITK_VMCNT(0));
    if (mine > 0) {
        u32x4 fa[MB][4], fb[NB][4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = mb * 32 + r;
                fa[mb][q] = *(const u32x4*)(dma_area + row * kChunkBytes + slot_of(row, 2 * q + h) * 16);
            }
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = BM + nb * 32 + r;
                fb[nb][q] = *(const u32x4*)(dma_area + row * kChunkBytes + slot_of(row, 2 * q + h) * 16);
            }
        }
        mfma_chunk(fa, fb, chunk_of(mine - 1));
    }

    // The partial tile goes into this wave's own DMA area, which no other
    // wave reads: no barrier before the writes, so early waves write while
    // late ones still multiply (measured ~0.3 us off the headline GEMM).
    sum_and_store<BM, BN, W, MB, NB, ROWS * kChunkBytes / 4>(reinterpret_cast<float*>(&dma_lds[0][0]), acc,
                                     P + ((size_t)s * M + (size_t)mt * BM) * N + (size_t)nt * BN, N,
                                     min(BN, N - nt * BN), wave, lane);
}

template <int DT, int BM, int BN, int W, int R>
hipError_t launch_wavek_dma(const void* A, const void* B, float* P, int64_t M, int64_t N, int64_t K,
                            int64_t kps, int64_t splits, int order, hipStream_t stream) {
    const int tiles_m = (int)(M / BM), tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * (int64_t)tiles_n * splits));
    const uint8_t* a = (const uint8_t*)A;
    const uint8_t* b = (const uint8_t*)B;
    int m = (int)M, n = (int)N, k = (int)K, kp = (int)kps;
    TileGrid tg = make_tile_grid(tiles_m, tiles_n, (int)splits, order);
    void* args[] = {&a, &b, &P, &m, &n, &k, &kp, &tg};
    return hipLaunchKernel((const void*)&gemm_bt_wavek_dma<DT, BM, BN, W, R>, grid, dim3(W * 64), args,
                           0, stream);
}

template <int DT, int BM, int BN, int W, int D, int BL>
hipError_t launch_wavek(const void* A, const void* B, float* P, int64_t M, int64_t N, int64_t K,
                        int64_t kps, int64_t splits, int order, hipStream_t stream) {
    const int tiles_m = (int)(M / BM), tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * (int64_t)tiles_n * splits));
    const dim3 block(W * 64);
    const uint8_t* a = (const uint8_t*)A;
    const uint8_t* b = (const uint8_t*)B;
    int m = (int)M, n = (int)N, k = (int)K, kp = (int)kps;
    TileGrid tg = make_tile_grid(tiles_m, tiles_n, (int)splits, order);
    void* args[] = {&a, &b, &P, &m, &n, &k, &kp, &tg};
    return hipLaunchKernel((const void*)&gemm_bt_wavek<DT, BM, BN, W, D, BL>, grid, block, args, 0,
                           stream);
}

// The instantiated configurations: (BM, BN, waves, stages).
// Instantiated (BM, BN, waves, register chunks) of the last-chunk-by-DMA kernel.
#define SPLITK_WAVEKDMA_CONFIGS(X) \
    X(32, 64, 8, 1)                \
    X(32, 32, 8, 1)                \
    X(32, 32, 8, 0)                \
    X(32, 64, 8, 0)

#define SPLITK_WAVEK_CONFIGS(X) \
    X(32, 32, 4, 1)             \
    X(32, 32, 4, 2)             \
    X(32, 32, 4, 4)             \
    X(32, 64, 4, 1)             \
    X(32, 64, 4, 2)             \
    X(32, 64, 4, 4)             \
    X(32, 32, 8, 1)             \
    X(32, 32, 8, 2)             \
    X(32, 64, 8, 1)             \
    X(32, 64, 8, 2)             \
    X(64, 64, 4, 2)             \
    X(64, 64, 4, 4)

// Instantiated configurations for B stored as [K,N]: the register-staged
// skinny kernel and the large-tile kernel (the DMA-tail skinny kernel
// transposes 32 B rows at a time, which has no counterpart when B's rows are
// k-rows).
#define SPLITK_KN_WAVEK_CONFIGS(X) \
    X(32, 32, 8, 1)                \
    X(32, 32, 8, 2)                \
    X(32, 64, 8, 1)                \
    X(32, 64, 8, 2)

#define SPLITK_KN_TILED_CONFIGS(X) \
    X(256, 256, 2, 2, 2)           \
    X(256, 128, 2, 2, 3)           \
    X(256, 128, 2, 4, 3)

template <int DT>
hipError_t launch_dtype_kn(const GemmPlan& p, const void* A, const void* B, float* P, int64_t M,
                           int64_t N, int64_t K, int64_t kps, int64_t splits, hipStream_t st) {
    if (p.kind == kWaveK) {
#define X(cbm, cbn, cw, cd)                                                    \
    if (p.bm == cbm && p.bn == cbn && p.waves == cw && p.stages == cd)        \
        return launch_wavek<DT, cbm, cbn, cw, cd, 1>(A, B, P, M, N, K, kps, splits, p.order, st);
        SPLITK_KN_WAVEK_CONFIGS(X)
#undef X
    }
    if (p.kind == kTiled && p.persist) {
#define X(cbm, cbn, cwm, cwn)                                                     \
    if (p.bm == cbm && p.bn == cbn && p.waves == cwm * cwn && p.stages == cwm)    \
        return launch_tiled_pt<DT, cbm, cbn, cwm, cwn, 1>(A, B, P, M, N, K, kps, splits, st);
        SPLITK_KN_TILED_PT_CONFIGS(X)
#undef X
        return hipErrorInvalidConfiguration;
    }
    if (p.kind == kTiled) {
#define X(cbm, cbn, cwm, cwn, cnb)                                                \
    if (p.bm == cbm && p.bn == cbn && p.waves == cwm * cwn && p.stages == cwm &&  \
        p.nbuf == cnb)                                                            \
        return launch_tiled<DT, cbm, cbn, cwm, cwn, cnb, 1>(A, B, P, M, N, K, kps, splits, p.order, st);
        SPLITK_KN_TILED_CONFIGS(X)
#undef X
    }
    return hipErrorInvalidConfiguration;
}

template <int DT>
hipError_t launch_dtype(const GemmPlan& p, const void* A, const void* B, float* P, int64_t M,
                        int64_t N, int64_t K, int64_t kps, int64_t splits, hipStream_t st) {
    if (p.layout == kLayoutKN) return launch_dtype_kn<DT>(p, A, B, P, M, N, K, kps, splits, st);
    if (p.kind == kWaveK) {
#define X(cbm, cbn, cw, cd)                                                    \
    if (p.bm == cbm && p.bn == cbn && p.waves == cw && p.stages == cd)        \
        return launch_wavek<DT, cbm, cbn, cw, cd, 0>(A, B, P, M, N, K, kps, splits, p.order, st);
        SPLITK_WAVEK_CONFIGS(X)
#undef X
    }
    if (p.kind == kWaveKDma) {
#define X(cbm, cbn, cw, cr)                                                     \
    if (p.bm == cbm && p.bn == cbn && p.waves == cw && p.stages == cr)          \
        return launch_wavek_dma<DT, cbm, cbn, cw, cr>(A, B, P, M, N, K, kps, splits, p.order, st);
        SPLITK_WAVEKDMA_CONFIGS(X)
#undef X
    }
    if (p.kind == kTiled && p.persist) {
#define X(cbm, cbn, cwm, cwn)                                                     \
    if (p.bm == cbm && p.bn == cbn && p.waves == cwm * cwn && p.stages == cwm)    \
        return launch_tiled_pt<DT, cbm, cbn, cwm, cwn, 0>(A, B, P, M, N, K, kps, splits, st);
        SPLITK_TILED_PT_CONFIGS(X)
#undef X
        return hipErrorInvalidConfiguration;
    }
    if (p.kind == kTiled) {
#define X(cbm, cbn, cwm, cwn, cnb)                                                \
    if (p.bm == cbm && p.bn == cbn && p.waves == cwm * cwn && p.stages == cwm &&  \
        p.nbuf == cnb)                                                            \
        return launch_tiled<DT, cbm, cbn, cwm, cwn, cnb, 0>(A, B, P, M, N, K, kps, splits, p.order, st);
        SPLITK_TILED_CONFIGS(X)
#undef X
    }
    return hipErrorInvalidConfiguration;
}

}  // namespace

bool wavekdma_config_exists(int bm, int bn, int w, int r) {
#define X(cbm, cbn, cw, cr) \
    if (bm == cbm && bn == cbn && w == cw && r == cr) return true;
    SPLITK_WAVEKDMA_CONFIGS(X)
#undef X
    return false;
}

bool wavek_config_exists(int layout, int bm, int bn, int w, int d) {
#define X(cbm, cbn, cw, cd) \
    if (bm == cbm && bn == cbn && w == cw && d == cd) return true;
    if (layout == kLayoutKN) {
        SPLITK_KN_WAVEK_CONFIGS(X)
        return false;
    }
    SPLITK_WAVEK_CONFIGS(X)
#undef X
    return false;
}

bool tiled_pt_config_exists(int layout, int bm, int bn, int wm, int wn) {
#define X(cbm, cbn, cwm, cwn) \
    if (bm == cbm && bn == cbn && wm == cwm && wn == cwn) return true;
    if (layout == kLayoutKN) {
        SPLITK_KN_TILED_PT_CONFIGS(X)
        return false;
    }
    SPLITK_TILED_PT_CONFIGS(X)
#undef X
    return false;
}

bool tiled_config_exists(int layout, int bm, int bn, int wm, int wn, int nbuf) {
#define X(cbm, cbn, cwm, cwn, cnb) \
    if (bm == cbm && bn == cbn && wm == cwm && wn == cwn && nbuf == cnb) return true;
    if (layout == kLayoutKN) {
        SPLITK_KN_TILED_CONFIGS(X)
        return false;
    }
    SPLITK_TILED_CONFIGS(X)
#undef X
    return false;
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
