"""Host-side tests of the C ABI: the library loads, exports what
include/splitk.h declares, and rejects every argument the launch contract
forbids ("Aligned shared rows for pipelined NAX on CUDA", section "Contract
and correctness") before launching anything.

No test here launches a kernel.  The pointer checks pass made-up addresses,
which the library must reject before any HIP call; they are skipped where a
GPU is present, and the GPU tests cover the same statuses with real buffers.
"""
from __future__ import annotations

import ctypes

import pytest

from conftest import gpu_available
from split_dense_gemm_amd import inputs

OK, NULL, DTYPE, SHAPE, SPLIT, ALIAS, ALIGN, RANGE, LAUNCH, WORKSPACE, PLAN, SCRATCH = range(12)

BF16 = inputs.DTYPE_CODES["bf16"]


def test_exports_every_declared_symbol(hip_lib):
    names = hip_lib.header_functions()
    assert set(names) == {"splitk_gemm_bt", "splitk_reduce", "splitk_gemm_bt_reduce",
                          "splitk_reduce_typed", "splitk_gemm_bt_reduce_typed",
                          "splitk_choose_splits", "splitk_gemm_bt_auto",
                          "splitk_gemm_bn", "splitk_gemm_bn_reduce", "splitk_describe_bn",
                          "splitk_status_str", "splitk_describe", "splitk_reduce_for_gemm",
                          "splitk_gemm_planned", "splitk_describe_planned",
                          "splitk_gemm_bt_auto_noalloc"}
    lib = hip_lib.load()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(hip_lib):
    lib = hip_lib.load()
    texts = [lib.splitk_status_str(s).decode() for s in range(12)]
    assert texts[0] == "ok" and len(set(texts)) == 12 and "unknown status" not in texts
    assert lib.splitk_status_str(99).decode() == "unknown status"


# (M, N, K, kps, splits, dtype) -> status from the shape and split checks
SHAPE_CASES = [
    ((256, 1024, 2048, 1024, 2, BF16), OK),
    ((32, 64, 64, 32, 2, 0), OK),
    ((32, 512, 2080, 544, 4, 1), OK),
    ((64, 128, 1056, 1024, 2, BF16), OK),     # last split of 32
    ((256, 1024, 2048, 1024, 2, 3), DTYPE),
    ((256, 1024, 2048, 1024, 2, -1), DTYPE),
    ((0, 64, 64, 32, 2, BF16), SHAPE),
    ((48, 64, 64, 32, 2, BF16), SHAPE),       # M not a multiple of 32
    ((32, 0, 64, 32, 2, BF16), SHAPE),        # N must be positive
    ((32, -64, 64, 32, 2, BF16), SHAPE),
    ((32, 64, 48, 48, 1, BF16), SHAPE),       # K not a multiple of 32
    ((32, 64, 64, 16, 4, BF16), SHAPE),       # kps not a multiple of 32
    ((32, 64, -64, 32, 2, BF16), SHAPE),
    ((32, 64, 2048, 512, 0, BF16), SPLIT),
    ((32, 64, 2048, 512, 3, BF16), SPLIT),    # splits do not cover K
    ((32, 64, 2048, 512, 5, BF16), SPLIT),    # fifth split would start at K
    ((32, 64, 2048, 4096, 2, BF16), SPLIT),   # second split would start past K
    ((32, 64, 2080, 544, 3, BF16), SPLIT),
    ((32, 64, 2**31, 2**31, 1, BF16), RANGE),
    ((2**20, 64, 2**12, 2**12, 1, BF16), RANGE),  # M*K = 2^32 elements
    ((2**16, 2**16, 32, 32, 1, BF16), RANGE),      # M*N = 2^32
    ((2**15, 2**15, 64, 32, 2, BF16), RANGE),      # splits*M*N = 2^31
]


@pytest.mark.parametrize("args,status", SHAPE_CASES)
def test_describe_checks_shape_and_split(hip_lib, args, status):
    buf = ctypes.create_string_buffer(128)
    got = hip_lib.load().splitk_describe(*args, buf, len(buf))
    assert got == status
    if status == OK:
        assert buf.value.split()[0] in (b"wavek", b"wavekdma", b"tiled")


def test_plan_for_each_workload(hip_lib):
    for w in inputs.WORKLOADS.values():
        text = hip_lib.describe(w.M, w.N, w.K, w.kps, w.splits, inputs.DTYPE_CODES[w.dtype])
        assert "grid" in text


A_PTR, B_PTR, P_PTR, C_PTR = 0x10000000, 0x20000000, 0x30000000, 0x40000000


@pytest.mark.skipif(gpu_available(), reason="made-up pointers are only passed where no GPU exists")
class TestPointerChecksWithoutDevice:
    def gemm(self, hip_lib, A=A_PTR, B=B_PTR, P=P_PTR, M=256, N=1024, K=2048, kps=1024, S=2, dt=BF16):
        return hip_lib.raw_call("splitk_gemm_bt", A, B, P, M, N, K, kps, S, dt, None)

    def fused(self, hip_lib, A=A_PTR, B=B_PTR, P=P_PTR, C=C_PTR, M=256, N=1024, K=2048, kps=1024,
              S=2, dt=BF16):
        return hip_lib.raw_call("splitk_gemm_bt_reduce", A, B, P, C, M, N, K, kps, S, dt, None)

    def test_null(self, hip_lib):
        assert self.gemm(hip_lib, A=None) == NULL
        assert self.gemm(hip_lib, B=None) == NULL
        assert self.gemm(hip_lib, P=None) == NULL
        assert self.fused(hip_lib, C=None) == NULL
        assert hip_lib.raw_call("splitk_reduce", None, C_PTR, 2, 256, 1024, None) == NULL
        assert hip_lib.raw_call("splitk_reduce", P_PTR, None, 2, 256, 1024, None) == NULL

    def test_alignment(self, hip_lib):
        assert self.gemm(hip_lib, A=A_PTR + 8) == ALIGN
        assert self.gemm(hip_lib, B=B_PTR + 2) == ALIGN
        assert self.gemm(hip_lib, P=P_PTR + 4) == ALIGN
        assert self.fused(hip_lib, C=C_PTR + 4) == ALIGN
        assert hip_lib.raw_call("splitk_reduce", P_PTR + 4, C_PTR, 2, 256, 1024, None) == ALIGN

    def test_aliasing(self, hip_lib):
        a_bytes = 256 * 2048 * 2
        assert self.gemm(hip_lib, P=A_PTR) == ALIAS
        assert self.gemm(hip_lib, P=A_PTR + a_bytes - 16) == ALIAS        # tail overlap
        assert self.gemm(hip_lib, P=B_PTR - 16) == ALIAS                   # head overlap
        p_bytes = 2 * 256 * 1024 * 4
        assert self.fused(hip_lib, C=P_PTR + p_bytes - 16) == ALIAS
        assert self.fused(hip_lib, C=A_PTR) == ALIAS
        assert hip_lib.raw_call("splitk_reduce", P_PTR, P_PTR + 1024, 2, 256, 1024, None) == ALIAS

    def test_typed_output_checks(self, hip_lib):
        call = lambda *a: hip_lib.raw_call("splitk_reduce_typed", *a)  # noqa: E731
        assert call(P_PTR, C_PTR, 2, 256, 1024, 3, None) == DTYPE
        assert call(P_PTR, C_PTR, 2, 256, 1024, -1, None) == DTYPE
        assert call(None, C_PTR, 2, 256, 1024, 1, None) == NULL
        assert call(P_PTR, C_PTR + 8, 2, 256, 1024, 2, None) == ALIGN
        # A 16-bit C of M*N elements ends M*N*2 bytes after its start.
        p_bytes = 2 * 256 * 1024 * 4
        assert call(P_PTR, P_PTR + p_bytes - 16, 2, 256, 1024, 1, None) == ALIAS
        fused = lambda *a: hip_lib.raw_call("splitk_gemm_bt_reduce_typed", *a)  # noqa: E731
        assert fused(A_PTR, B_PTR, P_PTR, C_PTR, 256, 1024, 2048, 1024, 2, BF16, 5, None) == DTYPE
        assert fused(A_PTR, B_PTR, P_PTR, A_PTR + 16, 256, 1024, 2048, 1024, 2, BF16, 1, None) == ALIAS

    def test_auto_checks(self, hip_lib):
        def auto(A=A_PTR, B=B_PTR, W=P_PTR, wn=1 << 30, C=C_PTR, M=256, N=1024, K=2048, dt=BF16, ot=0):
            return hip_lib.raw_call("splitk_gemm_bt_auto", A, B, W, wn, C, M, N, K, dt, ot, None)
        assert auto(C=None) == NULL
        assert auto(A=None) == NULL
        assert auto(ot=7) == DTYPE
        assert auto(M=48) == SHAPE
        # Workspace: too small is its own status; NULL with a need is NULL.
        kps, s, need = hip_lib.choose_splits(32, 512, 16384, BF16)
        assert s > 1 and need == s * 32 * 512
        assert auto(M=32, N=512, K=16384, wn=need - 1) == WORKSPACE
        assert auto(M=32, N=512, K=16384, W=None, wn=need) == NULL
        assert auto(M=32, N=512, K=16384, wn=need, W=P_PTR + 4) == ALIGN
        assert auto(M=32, N=512, K=16384, wn=need, W=A_PTR) == ALIAS
        assert auto(M=32, N=512, K=16384, wn=need, C=P_PTR + 16) == ALIAS
        # One split with an F32 C needs no workspace; C must not overlap A or B.
        kps, s, need = hip_lib.choose_splits(4096, 8192, 1024, BF16)
        assert (s, need) == (1, 0)
        assert auto(M=4096, N=8192, K=1024, W=None, wn=0, C=A_PTR) == ALIAS
        assert auto(M=4096, N=8192, K=1024, W=None, wn=0, C=C_PTR + 8) == ALIGN

    def test_shape_errors_come_before_pointer_checks(self, hip_lib):
        assert self.gemm(hip_lib, A=A_PTR + 8, M=48) == SHAPE
        assert self.gemm(hip_lib, P=A_PTR, S=3) == SPLIT
        assert hip_lib.raw_call("splitk_reduce", P_PTR, C_PTR, 0, 256, 1024, None) == SPLIT
        assert hip_lib.raw_call("splitk_reduce", P_PTR, C_PTR, 2, 256, 0, None) == SHAPE
        assert hip_lib.raw_call("splitk_reduce", P_PTR, C_PTR, 2, 48, 64, None) == SHAPE


def test_binding_rejects_host_tensors(hip_lib):
    import torch

    a = torch.zeros(32, 64, dtype=torch.bfloat16)
    b = torch.zeros(64, 64, dtype=torch.bfloat16)
    p = torch.zeros(2, 32, 64)
    with pytest.raises(ValueError):
        hip_lib.gemm_bt(a, b, p, 32, 2)


# ------------------------------------------------ automatic split count
# Host logic only: the choice among the sampled split counts of "Aligned
# shared rows for pipelined NAX on CUDA", section "Measurement protocol".

CHOICE_SHAPES = [(m, n, k) for m in (32, 96, 256, 1024, 4096) for n in (64, 512, 4096, 8192)
                 for k in (32, 96, 1024, 2080, 16384)]


@pytest.mark.parametrize("dt", [0, 1, 2])
@pytest.mark.parametrize("ot", [0, 1, 2])
def test_choice_is_a_valid_geometry(hip_lib, dt, ot):
    for M, N, K in CHOICE_SHAPES:
        kps, s, need = hip_lib.choose_splits(M, N, K, dt, ot)
        assert s in (1, 2, 4, 8, 16), (M, N, K, s)
        assert kps % 32 == 0 and (s - 1) * kps < K <= s * kps, (M, N, K, kps, s)
        assert need == (0 if (s == 1 and ot == 0) else s * M * N)
        if dt != 0 and K % 64 == 0 and s > 1:
            assert kps % 64 == 0, "16-bit splits should hold whole 128-byte chunks"
        assert hip_lib.describe(M, N, K, kps, s, dt)  # the GEMM accepts it
        assert hip_lib.choose_splits(M, N, K, dt, ot) == (kps, s, need)  # deterministic


def test_choice_follows_the_measured_extremes(hip_lib):
    # Decided by wide margins in MI355X measurements of the chain
    # (e.g. 82 us with one split against 200 us with two for the first).
    assert hip_lib.choose_splits(4096, 8192, 1024, BF16)[1] == 1
    assert hip_lib.choose_splits(2048, 8192, 8192, BF16)[1] == 1
    assert hip_lib.choose_splits(32, 512, 16384, BF16)[1] >= 4
    assert hip_lib.choose_splits(512, 8192, 16384, BF16)[1] >= 2
    assert hip_lib.choose_splits(256, 8192, 8192, BF16)[1] >= 2
    # Short K leaves nothing to split.
    assert hip_lib.choose_splits(256, 1024, 32, BF16)[1] == 1


@pytest.mark.parametrize("args,status", [
    ((48, 512, 1024, BF16, 0), SHAPE), ((32, 0, 1024, BF16, 0), SHAPE),
    ((32, 512, 1000, BF16, 0), SHAPE), ((32, 512, 0, BF16, 0), SHAPE),
    ((32, 512, 1024, 3, 0), DTYPE), ((32, 512, 1024, BF16, 9), DTYPE),
    ((1 << 16, 64, 1 << 15, BF16, 0), RANGE),
])
def test_choice_checks(hip_lib, args, status):
    out = [ctypes.c_int64() for _ in range(3)]
    assert hip_lib.load().splitk_choose_splits(*args, *[ctypes.byref(o) for o in out]) == status
    assert hip_lib.load().splitk_choose_splits(32, 512, 1024, BF16, 0, None, ctypes.byref(out[1]),
                                               ctypes.byref(out[2])) == NULL


# ------------------------------------------------ B stored [K,N]

# N tails: any positive N with B stored [N,K]; a multiple of 8 with [K,N].
N_TAIL_CASES = [(N, OK, OK if N % 8 == 0 else SHAPE) for N in (1, 3, 8, 36, 40, 96, 100, 1000, 1030)]


@pytest.mark.parametrize("N,status_nk,status_kn", N_TAIL_CASES)
def test_n_tails_accepted(hip_lib, N, status_nk, status_kn):
    buf = ctypes.create_string_buffer(128)
    lib = hip_lib.load()
    assert lib.splitk_describe(64, N, 1024, 256, 4, BF16, buf, len(buf)) == status_nk
    assert lib.splitk_describe_bn(64, N, 1024, 256, 4, BF16, buf, len(buf)) == status_kn
    if status_nk == OK:
        kps, s, need = hip_lib.choose_splits(64, N, 1024, BF16)
        assert (s - 1) * kps < 1024 <= s * kps


def test_tail_tiles_in_plans(hip_lib):
    # Column tiles are counted with the narrowed last tile included: 16-bit
    # inputs take 256x256 tiles by the same rules as an N that 256 divides
    # (persistent over several rounds of short splits) ...
    assert hip_lib.describe_bn(2048, 4000, 1024, 256, 4, BF16) == (
        "tiled bm256 bn256 waves2x2 ring2 block256 grid256 persistent")
    assert hip_lib.describe(2048, 4000, 1024, 256, 4, BF16) == (
        "tiled bm256 bn256 waves2x2 ring2 block256 grid256 persistent")
    assert hip_lib.describe(2048, 2000, 4096, 1024, 4, BF16) == (
        f"tiled bm256 bn256 waves2x2 ring2 block256 grid{8 * 8 * 4}")
    # ... and 256x128 tiles where the last round of 256x256 ones would be at
    # most half full (B as [N,K]): 384 of them in two splits.
    text = hip_lib.describe(4096, 3000, 2048, 1024, 2, BF16)
    assert text.startswith("tiled bm256 bn128") and text.endswith(f"grid{16 * 24 * 2}"), text
    assert hip_lib.describe_bn(4096, 3000, 2048, 1024, 2, BF16) == (
        "tiled bm256 bn256 waves2x2 ring2 block256 grid256 persistent")
    assert hip_lib.describe_bn(4096, 3944, 2048, 2048, 1, BF16) == (
        f"tiled bm256 bn256 waves2x2 ring2 block256 grid{16 * 16}")  # one round
    # F32 keeps 256x256 tiles to an N that 256 divides.
    assert " bn256 " not in hip_lib.describe(2048, 4000, 1024, 256, 4, 0)
    text = hip_lib.describe(64, 100, 1024, 256, 4, BF16)
    assert f" grid{2 * (2 if ' bn64 ' in text else 4) * 4}" in text, text


def test_tile_order_choice(hip_lib):
    """Skinny plans put every split of a tile on one XCD ("splitfast") only
    while the operand panels of the tiles one XCD holds at once stay within
    3 MiB of its L2; large tiles, long K and shapes the tile-ordered slab sum
    cannot serve (N % 4 != 0, more than eight splits) keep the split-major
    order."""
    fast = [(256, 1024, 2048, 1024, 2), (512, 1024, 2048, 1024, 2), (96, 512, 2048, 512, 4),
            (64, 256, 2048, 256, 8)]
    major = [(64, 768, 12288, 1536, 8), (192, 768, 6144, 3072, 2), (192, 3072, 12288, 3072, 4),
             (64, 130, 512, 256, 2), (32, 64, 2048, 128, 16), (2048, 4096, 4096, 512, 8)]
    for shape in fast:
        assert hip_lib.describe(*shape, BF16).endswith(" splitfast"), shape
    for shape in major:
        assert "splitfast" not in hip_lib.describe(*shape, BF16), shape


def test_large_tile_order_choice(hip_lib):
    """256-row tiles take the split-fastest order only on a grid of one round
    (at most 256 workgroups on 256 CUs) with at most 32 MiB of slabs and at
    most 12 chunks of 128 bytes per split, for both B layouts."""
    fast = [(768, 1536, 1536, 384, 4), (512, 1536, 1536, 192, 8), (2048, 2048, 1024, 512, 2),
            (768, 3072, 1536, 768, 2)]
    major = [(768, 768, 12288, 1536, 8),    # 24 chunks per split
             (1536, 1536, 3072, 768, 4),    # 288 workgroups
             (2048, 4096, 1024, 512, 2),    # 64 MiB of slabs
             (768, 1536, 1536, 96, 16)]     # more than eight splits
    for describe in (hip_lib.describe, hip_lib.describe_bn):
        for shape in fast:
            text = describe(*shape, BF16)
            assert text.startswith("tiled bm256") and text.endswith(" splitfast"), (shape, text)
        for shape in major:
            text = describe(*shape, BF16)
            assert text.startswith("tiled bm256") and "splitfast" not in text, (shape, text)
    # F32: 32 elements per chunk, so 384 per split is 12 chunks and 416 is 13.
    text = hip_lib.describe(768, 1536, 1536, 384, 4, 0)
    assert text.startswith("tiled bm256") and text.endswith(" splitfast"), text
    text = hip_lib.describe(768, 1536, 1664, 416, 4, 0)
    assert text.startswith("tiled bm256") and "splitfast" not in text, text


@pytest.mark.parametrize("args,status", SHAPE_CASES)
def test_describe_bn_checks_shape_and_split(hip_lib, args, status):
    buf = ctypes.create_string_buffer(128)
    assert hip_lib.load().splitk_describe_bn(*args, buf, len(buf)) == status


def test_bn_plans_never_use_the_dma_tail_kernel(hip_lib):
    for M, N, K, kps, S in [(32, 512, 2048, 512, 4), (256, 1024, 2048, 1024, 2),
                            (2048, 4096, 4096, 512, 8), (96, 512, 2048, 512, 4)]:
        text = hip_lib.describe_bn(M, N, K, kps, S, BF16)
        assert text.startswith(("wavek ", "tiled ")), text


@pytest.mark.skipif(gpu_available(), reason="made-up pointers are only passed where no GPU exists")
def test_bn_pointer_checks_without_device(hip_lib):
    bn = lambda *a: hip_lib.raw_call("splitk_gemm_bn", *a)  # noqa: E731
    assert bn(A_PTR, None, P_PTR, 256, 1024, 2048, 1024, 2, BF16, None) == NULL
    assert bn(A_PTR, B_PTR + 4, P_PTR, 256, 1024, 2048, 1024, 2, BF16, None) == ALIGN
    assert bn(A_PTR, B_PTR, B_PTR + 64, 256, 1024, 2048, 1024, 2, BF16, None) == ALIAS
    assert bn(A_PTR, B_PTR, P_PTR, 256, 1024, 2048, 1024, 3, BF16, None) == SPLIT
    red = lambda *a: hip_lib.raw_call("splitk_gemm_bn_reduce", *a)  # noqa: E731
    assert red(A_PTR, B_PTR, P_PTR, None, 256, 1024, 2048, 1024, 2, BF16, 0, None) == NULL
    assert red(A_PTR, B_PTR, P_PTR, C_PTR, 256, 1024, 2048, 1024, 2, BF16, 4, None) == DTYPE
    assert red(A_PTR, B_PTR, P_PTR, A_PTR, 256, 1024, 2048, 1024, 2, BF16, 0, None) == ALIAS


def test_short_last_round_takes_256x128_tiles(hip_lib):
    """With B as [N,K], 256x128 tiles replace 256x256 ones where the last
    round of 256x256 workgroups would be at most half full: for 16-bit inputs
    in one or two splits with 257-384 workgroups or with at most 12 chunks
    per split.  F32 takes the tile that packs the rounds best, 128x128
    included with B as [N,K].  Otherwise 256x256 tiles stay, and always for
    16-bit inputs with B as [K,N]."""
    half = [(4096, 4608, 4096, 4096, 1), (3072, 6144, 1536, 1536, 1), (2048, 6144, 3072, 1536, 2)]
    full = [(2048, 4096, 4096, 512, 8), (4096, 4096, 8192, 2048, 4), (2048, 7168, 2048, 1024, 2),
            (3072, 6144, 12288, 3072, 4), (768, 3072, 12288, 1536, 8), (4096, 4096, 4096, 4096, 1)]
    for shape in half:
        wg = (shape[0] // 256) * (shape[1] // 256) * shape[4]
        assert 256 < wg <= 384 and shape[4] <= 2, shape
        assert hip_lib.describe(*shape, BF16).startswith(f"tiled bm256 bn128 waves2x4 ring3 block512 grid{2 * wg}")
        assert hip_lib.describe_bn(*shape, BF16).startswith(f"tiled bm256 bn256 waves2x2 ring2 block256 grid{wg}")
    for shape in full:
        wg = (shape[0] // 256) * (shape[1] // 256) * shape[4]
        assert not (256 < wg <= 384 and shape[4] <= 2), shape
        # Several rounds of splits of at most 16 chunks run persistently on
        # 256 workgroups (both B layouts).
        persistent = wg > 256 and shape[3] * 2 // 128 <= 16
        want = ("tiled bm256 bn256 waves2x2 ring2 block256 grid256 persistent" if persistent
                else f"tiled bm256 bn256 waves2x2 ring2 block256 grid{wg}")
        assert hip_lib.describe(*shape, BF16) == want, shape
        assert hip_lib.describe_bn(*shape, BF16) == want, shape
    # F32: the tile with the fewest rounds x tile area x per-tile factor
    # (256x256 1, 256x128 1.05, 128x128 1.1) among the three (B as [K,N]: no
    # 128x128); the same shapes in BF16 (24 chunks per split) keep 256x256.
    f32 = [((3072, 3072, 12288, 1536, 8), "bm256 bn128 waves2x4 ring3 block512 grid2304",
            "bm256 bn128 waves2x4 ring3 block512 grid2304", 1152),
           ((3072, 3072, 6144, 1536, 4), "bm128 bn128 waves2x2 ring4 block256 grid2304",
            "bm256 bn128 waves2x4 ring3 block512 grid1152", 576),
           ((2048, 4096, 4096, 1024, 4), "bm256 bn256 waves2x2 ring2 block256 grid512",
            "bm256 bn256 waves2x2 ring2 block256 grid512", 512)]
    for shape, plan_nk, plan_kn, wg in f32:
        assert hip_lib.describe(*shape, 0) == f"tiled {plan_nk}", shape
        assert hip_lib.describe_bn(*shape, 0) == f"tiled {plan_kn}", shape
        grid = "grid256 persistent" if shape[3] * 2 // 128 <= 16 else f"grid{wg}"
        assert hip_lib.describe(*shape, BF16) == f"tiled bm256 bn256 waves2x2 ring2 block256 {grid}", shape
    # F32 on 288 256x128 workgroups (144 256x256 ones): 128x128 tiles.
    assert hip_lib.describe(2048, 4608, 8192, 8192, 1, 0) == "tiled bm128 bn128 waves2x2 ring4 block256 grid576"
    # 16-bit, 1152 workgroups in 8 splits: 12 chunks per split switch, 24 do not.
    assert hip_lib.describe(3072, 3072, 6144, 768, 8, BF16).startswith("tiled bm256 bn128 waves2x4 ring3 block512 grid2304")
    assert hip_lib.describe(3072, 3072, 12288, 1536, 8, BF16).startswith("tiled bm256 bn256 waves2x2 ring2 block256 grid1152")


def test_persistent_large_tiles_rule(hip_lib):
    """256x256 tiles run persistently (one workgroup per CU walking several
    tiles), with either B layout, where there are more tiles than CUs and
    every split is at most 16 chunks; one round, longer splits and the other
    tiles keep one workgroup per tile."""
    yes = [((2048, 4096, 4096, 512, 8), BF16), ((2048, 4096, 4096, 512, 8), 1),
           ((2048, 4096, 4096, 512, 8), 0), ((2048, 4096, 4096, 1024, 4), BF16),
           ((4096, 4096, 4096, 256, 16), BF16)]
    no = [((4096, 4096, 8192, 2048, 4), BF16),   # 32 chunks per split
          ((2048, 4096, 4096, 1024, 4), 0),       # F32: 32 chunks per split
          ((4096, 4096, 4096, 4096, 1), BF16),    # one round
          ((256, 1024, 2048, 1024, 2), BF16)]     # skinny
    for shape, dt in yes:
        assert hip_lib.describe(*shape, dt).endswith("grid256 persistent"), (shape, dt)
        assert hip_lib.describe_bn(*shape, dt).endswith("grid256 persistent"), (shape, dt)
    for shape, dt in no:
        assert "persistent" not in hip_lib.describe(*shape, dt), (shape, dt)
        assert "persistent" not in hip_lib.describe_bn(*shape, dt), (shape, dt)
    # Named: "tiledp" is the persistent form, "tiled" never is; fewer tiles
    # than CUs launch one workgroup per tile.
    assert hip_lib.describe_planned("tiled,256,256,2,2", 2048, 4096, 4096, 512, 8, BF16).endswith("grid1024")
    assert hip_lib.describe_planned("tiledp,256,256,2,2", 2048, 4096, 4096, 512, 8, BF16).endswith(
        "grid256 persistent")
    assert hip_lib.describe_planned("tiledp,256,128,2,4", 512, 1024, 2048, 256, 8, BF16).endswith(
        "grid128 persistent")


# Named configurations (splitk_describe_planned / splitk_gemm_planned): text
# that names no instantiated configuration, a row tile that does not divide
# M, a DMA-tail kernel whose waves cannot hold a split, or an unknown layout
# are refused with SPLITK_ERR_PLAN; the shape checks come first.
PLAN_CASES = [
    ("wavek,32,64,8,2", 0, (256, 1024, 2048, 1024, 2, BF16), OK),
    ("tiled,256,128,2,4", 0, (512, 1024, 2048, 1024, 2, BF16), OK),
    ("tiled,256,128,2,4,3", 1, (512, 1024, 2048, 1024, 2, BF16), OK),
    ("wavekdma,32,64,8,1", 0, (256, 1024, 2048, 1024, 2, BF16), OK),
    ("wavekdma,32,64,8,1", 0, (256, 1024, 4096, 2048, 2, BF16), PLAN),   # 32 chunks > 8 x 2
    ("wavekdma,32,64,8,1", 1, (256, 1024, 2048, 1024, 2, BF16), PLAN),   # no [K,N] form
    ("tiled,256,256,2,2", 0, (128, 1024, 2048, 1024, 2, BF16), PLAN),    # 256 does not divide M
    ("wavek,32,64,8,3", 0, (256, 1024, 2048, 1024, 2, BF16), PLAN),      # not instantiated
    ("tiled,128,128,2,2", 1, (256, 1024, 2048, 1024, 2, BF16), PLAN),    # not for [K,N]
    ("tiled,256,256,2,2,5", 0, (512, 1024, 2048, 1024, 2, BF16), PLAN),  # ring depth not built
    ("wavek", 0, (256, 1024, 2048, 1024, 2, BF16), PLAN),
    ("", 0, (256, 1024, 2048, 1024, 2, BF16), PLAN),
    ("wavek,32,64,8,2", 2, (256, 1024, 2048, 1024, 2, BF16), PLAN),      # unknown layout
    ("wavek,32,64,8,2", 0, (48, 1024, 2048, 1024, 2, BF16), SHAPE),      # shape checks first
    ("wavek,32,64,8,2", 0, (256, 1024, 2048, 1024, 3, BF16), SPLIT),
    ("tiledp,256,256,2,2", 0, (2048, 4096, 4096, 512, 8, BF16), OK),
    ("tiledp,256,128,2,4", 0, (512, 1024, 2048, 256, 8, BF16), OK),
    ("tiledp,256,256,2,2", 1, (2048, 4096, 4096, 512, 8, BF16), OK),     # [K,N] form
    ("tiledp,256,128,2,4", 1, (512, 1024, 2048, 256, 8, BF16), PLAN),    # no [K,N] 256x128 form
    ("tiledp,256,256,2,2,2", 0, (2048, 4096, 4096, 512, 8, BF16), PLAN), # no ring argument
    ("tiledp,128,128,2,2", 0, (2048, 4096, 4096, 512, 8, BF16), PLAN),   # not instantiated
    ("tiledp,256,256,2,2", 0, (256, 512, 2048, 1024, 2, BF16), PLAN),    # 4 tiles: an XCD without one
]


@pytest.mark.parametrize("plan,layout,args,status", PLAN_CASES)
def test_describe_planned_statuses(hip_lib, plan, layout, args, status):
    buf = ctypes.create_string_buffer(128)
    got = hip_lib.load().splitk_describe_planned(plan.encode(), layout, *args, buf, len(buf))
    assert got == status, (plan, layout, args, buf.value)
    if status == OK:
        kind = plan.split(",")[0]
        text = buf.value.decode()
        assert text.startswith(kind.rstrip("p") + " ") and text.endswith(" persistent") == (kind == "tiledp"), text


def test_describe_planned_null_plan(hip_lib):
    buf = ctypes.create_string_buffer(128)
    assert hip_lib.load().splitk_describe_planned(None, 0, 256, 1024, 2048, 1024, 2, BF16, buf,
                                                  len(buf)) == NULL


def test_named_plan_keeps_the_tile_order_rule(hip_lib):
    """A named configuration takes the tile order the library would give it."""
    text = hip_lib.describe_planned("wavek,32,64,8,2", 256, 1024, 2048, 1024, 2, BF16)
    assert text.endswith(" splitfast"), text
    text = hip_lib.describe_planned("wavek,32,64,8,2", 256, 1024, 2048, 128, 16, BF16)
    assert "splitfast" not in text, text


@pytest.mark.skipif(gpu_available(), reason="made-up pointers are only safe without a GPU")
def test_gemm_planned_statuses_without_gpu(hip_lib):
    lib = hip_lib.load()
    A, B, P, C = 1 << 32, 2 << 32, 3 << 32, 4 << 32
    args = (256, 1024, 2048, 1024, 2, BF16, 0, None)
    assert lib.splitk_gemm_planned(None, 0, A, B, P, C, *args) == NULL
    assert lib.splitk_gemm_planned(b"wavek,32,64,8,3", 0, A, B, P, C, *args) == PLAN
    assert lib.splitk_gemm_planned(b"wavek,32,64,8,2", 0, A + 4, B, P, C, *args) == ALIGN
    assert lib.splitk_gemm_planned(b"wavek,32,64,8,2", 0, A, B, A, C, *args) == ALIAS
    assert lib.splitk_gemm_planned(b"wavek,32,64,8,2", 0, None, B, P, C, *args) == NULL
