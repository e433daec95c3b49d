/*
 * splitk.h -- C ABI of the split-K GEMM library for AMD MI355X (gfx950).
 *
 * Operation (restated from "Aligned shared rows for pipelined NAX on CUDA",
 * section "Contract and correctness", and "Wider consecutive-weight NAX
 * GEMM", section "Launch contract and correctness"):
 *
 *   A is [M,K] and B is [N,K], both row-major (each row contiguous in k), with
 *   elements of one type: F32, F16 or BF16.  B holds weights the caller has
 *   prepared once and keeps resident; the library reads it in place and never
 *   copies, packs or transposes it ("Performance method" of the second page).
 *   The K axis is cut into `splits` slices: slice s is
 *   [s*k_per_split, min((s+1)*k_per_split, K)).  Every slice starts below K,
 *   together they cover K, and only the last one may be shorter.
 *
 *   splitk_gemm_bt:  partials[s,i,j] = sum_{k in slice s} A[i,k] * B[j,k]
 *                    (F32 result; F16/BF16 products use the matrix cores'
 *                    native F16/BF16 inputs with F32 accumulation).
 *   splitk_reduce:   C[i,j] = sum_{s=0}^{splits-1} partials[s,i,j]
 *                    (F32, slabs added in ascending s).
 *   splitk_gemm_bt_reduce: the two above, back to back on one stream.
 *
 * Shape domain (same sections): M, K and k_per_split are positive multiples
 * of 32.  The pages also require N to be a multiple of 64; this library
 * accepts any positive N (the last column tile is narrowed: B rows past N are
 * never read and output columns past N never written).  Inputs have exactly the stated
 * extents -- the library never reads past A[M*K] or B[N*K] and never writes
 * outside partials[splits*M*N] or C[M*N] -- and outputs are separate storage
 * that aliases nothing else.
 *
 * Layout of every buffer is dense row-major: A[M][K], B[N][K],
 * partials[splits][M][N] (slab stride M*N floats), C[M][N].
 *
 * Pointers are device pointers (HIP device memory of the current device);
 * `stream` is a hipStream_t (NULL = the legacy default stream).  The caller
 * owns and frees every buffer; the library allocates nothing, keeps no state
 * between calls and is safe to call from several threads.
 *
 * Errors: arguments are checked on the host before anything is enqueued; a
 * non-zero status other than SPLITK_ERR_LAUNCH means nothing was launched.
 * SPLITK_ERR_LAUNCH means the HIP runtime refused a launch: from a call that
 * enqueues two kernels (a GEMM and its accumulation pass) it can come after
 * the GEMM was already enqueued, and the partials then receive the GEMM's
 * result while C is left as it was.  SPLITK_OK means the kernels were
 * enqueued on `stream`; execution is asynchronous and a device fault would
 * surface at the caller's next synchronisation.  There is no host
 * synchronisation, allocation or stream query inside, so the calls may be
 * captured into a HIP graph.  On success every element of partials (and of C)
 * is overwritten; nothing past their ends is touched.
 */
#ifndef SPLITK_H
#define SPLITK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPLITK_F32 = 0,
    SPLITK_F16 = 1,
    SPLITK_BF16 = 2
} splitk_dtype;

typedef enum {
    SPLITK_OK = 0,
    SPLITK_ERR_NULL = 1,   /* a required pointer is NULL                            */
    SPLITK_ERR_DTYPE = 2,  /* dtype is not one of splitk_dtype                      */
    SPLITK_ERR_SHAPE = 3,  /* M, K, k_per_split not positive multiples of 32, N not */
                           /* positive (not a multiple of 8 for splitk_gemm_bn)     */
    SPLITK_ERR_SPLIT = 4,  /* splits < 1, a slice starting at or past K, or the     */
                           /* slices not covering K                                 */
    SPLITK_ERR_ALIAS = 5,  /* an output overlaps an input or the other output       */
    SPLITK_ERR_ALIGN = 6,  /* a base pointer is not 16-byte aligned                 */
    SPLITK_ERR_RANGE = 7,  /* a buffer holds 2^31 elements or more                  */
    SPLITK_ERR_LAUNCH = 8, /* the HIP runtime refused the launch                    */
    SPLITK_ERR_WORKSPACE = 9, /* workspace smaller than the chosen geometry needs   */
    SPLITK_ERR_PLAN = 10,  /* splitk_gemm_planned: the named configuration is not   */
                           /* instantiated or does not fit the problem              */
    SPLITK_ERR_SCRATCH = 11 /* splitk_gemm_bt_auto_noalloc: the slabs would exceed  */
                            /* the library's static array                           */
} splitk_status;

/* F32 elements of the library-owned slab array of splitk_gemm_bt_auto_noalloc
 * (64 MiB per GPU). */
#define SPLITK_STATIC_SLAB_FLOATS (16LL << 20)

/*
 * Split-K GEMM into F32 partial slabs (first page, "Contract and
 * correctness"; second page, "Launch contract and correctness").
 *   A         [M,K] elements of `dtype`, read only.
 *   B         [N,K] elements of `dtype`, read only, resident weights.
 *   partials  [splits,M,N] F32, written in full (no accumulation into it).
 *   dtype     a splitk_dtype value.
 * Returns a splitk_status.
 */
int splitk_gemm_bt(const void* A, const void* B, float* partials, int64_t M, int64_t N, int64_t K,
                   int64_t k_per_split, int64_t splits, int dtype, void* stream);

/*
 * The separate accumulation pass that turns the slabs into the final output
 * (first page, "Contract and correctness" and "Measurement protocol"; second
 * page, "Performance method").
 *   partials  [splits,M,N] F32, read only; `splits` must be the value that
 *             produced them.
 *   C         [M,N] F32, written in full.
 * M must be a positive multiple of 32 and N positive, as for the GEMM.
 * Returns a splitk_status.
 */
int splitk_reduce(const float* partials, float* C, int64_t splits, int64_t M, int64_t N,
                  void* stream);

/*
 * Complete operation: splitk_gemm_bt then splitk_reduce on the same stream,
 * the chain the pages time as one captured graph (first page, "Measurement
 * protocol").  Arguments as above; all of them are checked before either
 * kernel is enqueued, and C must not overlap partials, A or B.
 */
int splitk_gemm_bt_reduce(const void* A, const void* B, float* partials, float* C, int64_t M,
                          int64_t N, int64_t K, int64_t k_per_split, int64_t splits, int dtype,
                          void* stream);

/*
 * Typed final output: the same slab sum, formed in F32 and then rounded to
 * `out_dtype` (a splitk_dtype; round to nearest, ties to even).  This is the
 * step downstream of the accumulation pass that the per-type final-output
 * tolerances of the pages suggest (first page, "Contract and correctness";
 * second page, "Performance method": F32 1e-4, F16 2e-3, BF16 2e-2).
 *   C   [M,N] elements of out_dtype, written in full.
 * Other arguments and errors as for splitk_reduce; SPLITK_ERR_DTYPE for an
 * unknown out_dtype.
 */
int splitk_reduce_typed(const float* partials, void* C, int64_t splits, int64_t M, int64_t N,
                        int out_dtype, void* stream);

/*
 * The accumulation pass of splitk_reduce_typed for slabs that splitk_gemm_bt
 * or splitk_gemm_bn has written with this geometry (M, N, K, k_per_split,
 * splits, dtype).  The result is the same sum, bit for bit (first page,
 * "Contract and correctness": the separate elementwise accumulation); only
 * the order in which workgroups visit the plane differs.  Where the GEMM
 * ran with all the splits of a tile on one XCD (small tiles whose operand
 * panels fit that XCD's L2; 256-row tiles on a grid of one round with at
 * most 32 MiB of slabs and short splits), each workgroup takes one output
 * tile, or one band of it, and runs on the XCD that wrote that tile's slabs,
 * so it reads them from that XCD's L2 instead of from memory; otherwise it
 * is the flat pass.  The fused calls run this pass.
 *   partials, C, out_dtype   as for splitk_reduce_typed.
 *   K, k_per_split, dtype    the GEMM's, checked as for splitk_gemm_bt.
 * Returns the statuses of splitk_reduce_typed and of splitk_gemm_bt's shape
 * and split checks; nothing is enqueued on an error.
 */
int splitk_reduce_for_gemm(const float* partials, void* C, int64_t M, int64_t N, int64_t K,
                           int64_t k_per_split, int64_t splits, int dtype, int out_dtype,
                           void* stream);

/*
 * splitk_gemm_bt then splitk_reduce_typed on the same stream.  C is [M,N] of
 * out_dtype; all arguments are checked before either kernel is enqueued.
 */
int splitk_gemm_bt_reduce_typed(const void* A, const void* B, float* partials, void* C, int64_t M,
                                int64_t N, int64_t K, int64_t k_per_split, int64_t splits,
                                int dtype, int out_dtype, void* stream);

/*
 * Automatic split count.  The pages time each shape at the split counts
 * 1, 2, 4, 8 and 16 and keep the fastest (first page, "Measurement
 * protocol"; second page, "Performance method").  This call makes that
 * choice without running anything: it ranks the same candidates with a cost
 * model of this library's kernels on one MI355X (the GEMM's workgroup rounds
 * over 256 CUs and its HBM traffic, plus the accumulation pass) and returns
 * the cheapest valid geometry.
 *   k_per_split, splits  the chosen geometry (k_per_split a multiple of 32,
 *                        of 64 for F16/BF16 where K allows).
 *   workspace_elems      F32 elements splitk_gemm_bt_auto needs as workspace
 *                        for it: splits*M*N, or 0 when one split writes an
 *                        F32 C directly.
 *   out_dtype            the splitk_dtype of C (an F16/BF16 C always needs
 *                        the rounding pass, hence workspace).
 * Host only; deterministic for given arguments.  Returns SPLITK_ERR_NULL for a
 * NULL output pointer and otherwise the shape, dtype and range checks of
 * splitk_gemm_bt.
 */
int splitk_choose_splits(int64_t M, int64_t N, int64_t K, int dtype, int out_dtype,
                         int64_t* k_per_split, int64_t* splits, int64_t* workspace_elems);

/*
 * C = A * B^T with the geometry splitk_choose_splits picks.  With one split
 * and an F32 C the GEMM writes C directly and no accumulation pass runs
 * (the splits = 1 case of the pages' sampled grid); otherwise the slabs go
 * to `workspace` and the pass (typed as out_dtype) writes C.
 *   workspace        F32 device buffer of workspace_elems elements; may be
 *                    NULL when the chosen geometry needs none.  Its contents
 *                    are overwritten; it must not overlap A, B or C.
 *   C                [M,N] of out_dtype, written in full.
 * Returns SPLITK_ERR_WORKSPACE (nothing launched) when workspace_elems is
 * below the need splitk_choose_splits reports, else as splitk_gemm_bt_reduce.
 */
int splitk_gemm_bt_auto(const void* A, const void* B, float* workspace, int64_t workspace_elems,
                        void* C, int64_t M, int64_t N, int64_t K, int dtype, int out_dtype,
                        void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * operation of splitk_gemm_bt_auto, same choice of split count, same kernels
 * and so the same C bit for bit, but with the F32 slabs in a device array the
 * library owns instead of a caller workspace.  The array holds
 * SPLITK_STATIC_SLAB_FLOATS floats (64 MiB); every GPU the library runs on
 * gets its own copy when the library's code is loaded there and keeps it
 * until the process ends.  Its address is looked up once per device, on the
 * first call with that device current (the current device must be the one
 * `stream` runs on).  The call allocates nothing and frees nothing.
 *   C   [M,N] of out_dtype, written in full.
 * Every call on one GPU uses that GPU's one array, so calls that may overlap
 * on one GPU (other streams, other threads) race on it: serialise them.  The
 * array keeps the last call's slabs; no call needs it to start at zero.
 * Returns the statuses of splitk_gemm_bt_auto, and SPLITK_ERR_SCRATCH
 * (nothing launched) when the chosen geometry needs more than
 * SPLITK_STATIC_SLAB_FLOATS slab elements (splits*M*N; splitk_choose_splits
 * reports it as workspace_elems); SPLITK_ERR_LAUNCH if the array's address
 * cannot be obtained.
 */
int splitk_gemm_bt_auto_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                                int dtype, int out_dtype, void* stream);

/*
 * The same split-K GEMM with B stored [K,N] instead of [N,K]: row k of B holds
 * B[k,0..N-1] contiguously (n-major weights).  The pages prepare weights in
 * both orders ("Wider consecutive-weight NAX GEMM", section "Performance
 * method"); the operation is unchanged:
 *   partials[s,i,j] = sum_{k in slice s} A[i,k] * B[k,j].
 *   B   [K,N] elements of `dtype`, read only, resident weights.
 * Every other argument, the checks and the statuses are those of
 * splitk_gemm_bt (B still spans N*K elements), except that N must be a
 * multiple of 8 so that every row of B starts 16-byte aligned.
 */
int splitk_gemm_bn(const void* A, const void* B, float* partials, int64_t M, int64_t N, int64_t K,
                   int64_t k_per_split, int64_t splits, int dtype, void* stream);

/*
 * splitk_gemm_bn then the accumulation pass on the same stream, C [M,N] of
 * out_dtype (F32, or F16/BF16 rounded to nearest even as in
 * splitk_reduce_typed).  All arguments are checked before either kernel is
 * enqueued.
 */
int splitk_gemm_bn_reduce(const void* A, const void* B, float* partials, void* C, int64_t M,
                          int64_t N, int64_t K, int64_t k_per_split, int64_t splits, int dtype,
                          int out_dtype, void* stream);

/* Static text for a status code ("unknown status" for anything else). */
const char* splitk_status_str(int status);

/*
 * Describes, without launching anything, the GEMM kernel configuration the
 * library would use for these arguments: writes a NUL-terminated text such as
 * "wavek bm32 bn64 waves4 stages4 block256 grid256" into buf (at most `len` bytes, truncated).
 * Returns a splitk_status from the same argument checks as splitk_gemm_bt,
 * minus the pointer checks.
 */
int splitk_describe(int64_t M, int64_t N, int64_t K, int64_t k_per_split, int64_t splits,
                    int dtype, char* buf, int64_t len);

/* As splitk_describe, for splitk_gemm_bn (B stored [K,N]). */
int splitk_describe_bn(int64_t M, int64_t N, int64_t K, int64_t k_per_split, int64_t splits,
                       int dtype, char* buf, int64_t len);

/*
 * Test and tuning hook: the operation of splitk_gemm_bt (b_layout 0, B
 * [N,K]) or splitk_gemm_bn (b_layout 1, B [K,N]) with a named kernel
 * configuration instead of the library's own choice, so that every
 * instantiated configuration can be run and checked.  The result is the same
 * operation; only speed differs.  When C is not NULL the accumulation pass
 * the fused calls run follows on the same stream (C of out_dtype, as in
 * splitk_gemm_bt_reduce_typed); when it is NULL only the GEMM runs and
 * out_dtype is ignored.
 *   plan   NUL-terminated text, one of
 *            "wavek,BM,BN,WAVES,STAGES"      register-staged skinny kernel
 *            "wavekdma,BM,BN,WAVES,REGCHUNKS" skinny kernel, last chunk by
 *                                             LDS DMA (B [N,K] only)
 *            "tiled,BM,BN,WM,WN[,RING]"       large-tile kernel, RING LDS
 *                                             buffers (default: the tile's)
 *            "tiledp,BM,BN,WM,WN"            persistent large-tile kernel:
 *                                             at most one workgroup per CU,
 *                                             each walking several tiles
 *                                             (B [K,N]: 256x256 only)
 *          naming an instantiated configuration (the lists in gemm_bt.hip).
 * Every check of splitk_gemm_bt applies first.  Returns SPLITK_ERR_NULL for a
 * NULL plan, SPLITK_ERR_PLAN (nothing launched) if the text names no
 * instantiated configuration for this layout, its row tile BM does not
 * divide M, the DMA-tail kernel's waves cannot hold a split's chunks
 * (more than WAVES x (REGCHUNKS + 1) 128-byte chunks), or a persistent
 * configuration has fewer than 8 tiles (one per XCD).  Host state: none;
 * the text is read during the call only.
 */
int splitk_gemm_planned(const char* plan, int b_layout, const void* A, const void* B, float* partials,
                        void* C, int64_t M, int64_t N, int64_t K, int64_t k_per_split, int64_t splits,
                        int dtype, int out_dtype, void* stream);

/* As splitk_describe, for the configuration `plan` names (statuses as for
 * splitk_gemm_planned, minus the pointer checks). */
int splitk_describe_planned(const char* plan, int b_layout, int64_t M, int64_t N, int64_t K,
                            int64_t k_per_split, int64_t splits, int dtype, char* buf, int64_t len);

#ifdef __cplusplus
}
#endif

#endif /* SPLITK_H */
