"""Every instantiated GEMM kernel configuration against the binary64 reference.

The automatic plan picks one configuration per shape; these tests run each
instantiated one (named through splitk_gemm_planned) on a small problem that
spans several tiles, several chunks per wave, a steady-state pipeline pass
and a short final split whose last chunk is half empty for 16-bit inputs.
Acceptance as in test_gpu_parity.py (tolerances of "Aligned shared rows for
pipelined NAX on CUDA", section "Contract and correctness").

The configuration lists are read from the kernel source so that a newly
instantiated configuration is tested without editing this file.  The
configurations instantiated for B stored [K,N] run through splitk_gemm_bn
with the same operands, B handed over as the transpose of the [N,K] array.
"""
from __future__ import annotations

import os
import re

import numpy as np
import pytest
import torch

import oracle
from conftest import gpu_available
from split_dense_gemm_amd import inputs

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "split_dense_gemm_amd", "csrc", "gemm_bt.hip")


def _configs(macro):
    text = open(SRC).read()
    body = text[text.index(f"#define {macro}(X)"):]
    body = body[: body.index("\n\n")]
    found = [tuple(int(v) for v in m.split(",")) for m in re.findall(r"X\(([\d, ]+)\)", body)]
    assert found, f"no configurations found for {macro}"
    return found


WAVEK = _configs("SPLITK_WAVEK_CONFIGS")
WAVEKDMA = _configs("SPLITK_WAVEKDMA_CONFIGS")
TILED = _configs("SPLITK_TILED_CONFIGS")
KN_WAVEK = _configs("SPLITK_KN_WAVEK_CONFIGS")
KN_TILED = _configs("SPLITK_KN_TILED_CONFIGS")
TILED_PT = _configs("SPLITK_TILED_PT_CONFIGS")
KN_TILED_PT = _configs("SPLITK_KN_TILED_PT_CONFIGS")


def _shape(kind, cfg):
    """(M, N, K, kps, splits) for a configuration.  N leaves a narrowed last
    column tile of 40 columns (a multiple of 8, as B stored [K,N] needs)."""
    bm, bn = cfg[0], cfg[1]
    if kind == "wavek":
        # 37 chunks of 32 per split: odd, so 16-bit slices end in a half
        # chunk; more chunks than waves x stages, so the pipeline loops.
        return 3 * bm, max(2 * bn, 128) + 40, 2 * 1184 + 96, 1184, 3
    if kind == "wavekdma":
        # At most waves x (register chunks + 1) chunks per split (F32 chunks
        # hold 32 elements, 16-bit ones 64); odd multiples of 32 end 16-bit
        # slices in a half chunk, and the short last split leaves some waves
        # with fewer chunks than others.
        kps = 32 * (7 if cfg[3] == 0 else 15)
        return 3 * bm, max(2 * bn, 128) + 40, 2 * kps + 96, kps, 3
    return 2 * bm, 2 * bn + 40, 2 * 608 + 32, 608, 3


CASES = ([("nk", "wavek", c) for c in WAVEK] + [("nk", "wavekdma", c) for c in WAVEKDMA] +
         [("nk", "tiled", c) for c in TILED] + [("kn", "wavek", c) for c in KN_WAVEK] +
         [("kn", "tiled", c) for c in KN_TILED] + [("nk", "tiledp", c) for c in TILED_PT] +
         [("kn", "tiledp", c) for c in KN_TILED_PT])


def _plan_text(kind, cfg):
    """Plan text; tiled configurations also name their ring depth."""
    return f"{kind}," + ",".join(str(v) for v in cfg)


def _case_id(case):
    layout, kind, cfg = case
    return f"{layout}:{_plan_text(kind, cfg)}"


@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_named_plan_is_honoured(hip_lib, case):
    layout, kind, cfg = case
    M, N, K, kps, S = _shape(kind, cfg)
    text = hip_lib.describe_planned(_plan_text(kind, cfg), M, N, K, kps, S, 2, layout=layout)
    assert text.startswith(kind.rstrip("p")) and f"bm{cfg[0]} bn{cfg[1]}" in text, text
    assert text.endswith(" persistent") == (kind == "tiledp"), text
    if kind == "tiled":
        assert f"waves{cfg[2]}x{cfg[3]} ring{cfg[4]}" in text, text
    if kind == "tiledp":
        assert f"waves{cfg[2]}x{cfg[3]} ring2" in text, text


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="no GPU")
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=_case_id)
def test_config_parity(hip_lib, case, dtype):
    layout, kind, cfg = case
    plan = _plan_text(kind, cfg)
    M, N, K, kps, S = _shape(kind, cfg)
    print(f"case {layout}:{plan} {dtype} M{M} N{N} K{K} kps{kps} S{S}", flush=True)
    # B as the library receives it: [N,K], or its transpose stored [K,N].
    stored = (lambda t: t) if layout == "nk" else (lambda t: t.T.contiguous())
    dev = torch.device("cuda:0")
    a, b = inputs.make_operands(M, N, K, dtype, seed=sum(cfg[:4]),
                                zero_first_row=True, scale_last_row=True)
    a64 = oracle.decode(inputs.stored_bits(a), dtype)
    b64 = oracle.decode(inputs.stored_bits(b), dtype)
    RP, DP, _ = oracle.splitk_partials(a64, b64, kps, S)
    RC, DC, _ = oracle.gemm_bt(a64, b64)
    pbuf = inputs.guarded_buffer(S * M * N, "nan").to(dev)
    cbuf = inputs.guarded_buffer(M * N, "nan").to(dev)
    hip_lib.gemm_planned(plan, a.to(dev), stored(b).to(dev), pbuf[: S * M * N].view(S, M, N), kps, S,
                         C=cbuf[: M * N].view(M, N), layout=layout)
    torch.cuda.synchronize()
    p, c = pbuf.cpu().numpy(), cbuf.cpu().numpy()
    guard = np.float32(inputs.GUARD_VALUE).view(np.uint32)
    assert np.all(p[S * M * N:].view(np.uint32) == guard)
    assert np.all(c[M * N:].view(np.uint32) == guard)
    ep, _ = oracle.normalized_error(p[: S * M * N], RP, DP)
    ec, _ = oracle.normalized_error(c[: M * N], RC, DC)
    print(f"  partial err {ep:.3e}, final err {ec:.3e}", flush=True)
    assert ep <= 1e-4
    assert ec <= {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-2}[dtype]
    # Exact-arithmetic inputs: bit-for-bit.
    ea, eb = inputs.exact_operands(M, N, K, dtype, seed=7)
    ea64 = oracle.decode(inputs.stored_bits(ea), dtype)
    eb64 = oracle.decode(inputs.stored_bits(eb), dtype)
    EP, _, _ = oracle.splitk_partials(ea64, eb64, kps, S)
    P = torch.empty(S, M, N, device=dev)
    hip_lib.gemm_planned(plan, ea.to(dev), stored(eb).to(dev), P, kps, S, layout=layout)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(P.cpu().numpy().astype(np.float64), EP)


# Large-tile configurations on grids of more workgroups than the chip has CUs
# (6 x 6 tiles x 8 splits = 288): the first round starts staggered, later
# rounds reuse the freed CUs.  The last column tile is 40 columns wide, every
# full 16-bit split ends in a half chunk and the last split is short.  With
# exact-arithmetic inputs every partial and the final sum are exact, so both
# must match bit for bit (C is the binary64 sum of the exact partials).
MULTI_ROUND = ([("nk", "tiled", c, "bf16") for c in TILED] + [("kn", "tiled", c, "bf16") for c in KN_TILED] +
               [("nk", "tiled", TILED[0], "f16"), ("nk", "tiled", TILED[0], "f32")] +
               [("nk", "tiledp", c, "bf16") for c in TILED_PT] +
               [("nk", "tiledp", TILED_PT[0], "f16"), ("nk", "tiledp", TILED_PT[0], "f32")] +
               [("kn", "tiledp", c, dt) for c in KN_TILED_PT for dt in ("bf16", "f16", "f32")])


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="no GPU")
@pytest.mark.parametrize("case", MULTI_ROUND,
                         ids=lambda c: f"{c[0]}:{c[1]}," + ",".join(map(str, c[2])) + f"-{c[3]}")
def test_tiled_multi_round_exact(hip_lib, case):
    """On the persistent configurations the 288 tiles run on 256 workgroups:
    32 of them take a second tile, whose first two chunks are loaded while
    the first tile's partials are stored."""
    layout, kind, cfg, dtype = case
    bm, bn = cfg[0], cfg[1]
    M, N, S, kps = 6 * bm, 5 * bn + 40, 8, 96
    K = (S - 1) * kps + 64
    plan = _plan_text(kind, cfg)
    text = hip_lib.describe_planned(plan, M, N, K, kps, S, inputs.DTYPES[dtype], layout=layout)
    print(f"case {layout} {dtype} M{M} N{N} K{K} kps{kps} S{S}: {text}", flush=True)
    grid = "grid256 persistent" if kind == "tiledp" else "grid288"
    assert f"bm{bm} bn{bn}" in text and grid in text, text
    stored = (lambda t: t) if layout == "nk" else (lambda t: t.T.contiguous())
    dev = torch.device("cuda:0")
    ea, eb = inputs.exact_operands(M, N, K, dtype, seed=bm + bn + S)
    ea64 = oracle.decode(inputs.stored_bits(ea), dtype)
    eb64 = oracle.decode(inputs.stored_bits(eb), dtype)
    EP, _, _ = oracle.splitk_partials(ea64, eb64, kps, S)
    EC = EP.sum(axis=0)
    pbuf = inputs.guarded_buffer(S * M * N, "nan").to(dev)
    cbuf = inputs.guarded_buffer(M * N, "nan").to(dev)
    hip_lib.gemm_planned(plan, ea.to(dev), stored(eb).to(dev), pbuf[: S * M * N].view(S, M, N), kps, S,
                         C=cbuf[: M * N].view(M, N), layout=layout)
    torch.cuda.synchronize()
    p, c = pbuf.cpu().numpy(), cbuf.cpu().numpy()
    guard = np.float32(inputs.GUARD_VALUE).view(np.uint32)
    assert np.all(p[S * M * N:].view(np.uint32) == guard)
    assert np.all(c[M * N:].view(np.uint32) == guard)
    np.testing.assert_array_equal(p[: S * M * N].astype(np.float64), EP.reshape(-1))
    np.testing.assert_array_equal(c[: M * N].astype(np.float64), EC.reshape(-1))


# Large-tile configurations on one round of workgroups with few slabs: every
# split of a tile runs on one XCD (split fastest) and the slab sum takes each
# tile on that XCD.  Tile counts of 12 and 9 per split (one a multiple of 8
# XCDs' worth of tiles, one not), a 40-column last tile, 2, 5 and 8 splits,
# F32 and rounded BF16 / F16 outputs, both B layouts.  Exact-arithmetic
# inputs: the partials and C match the binary64 reference bit for bit (C
# rounded once).
SPLIT_FAST = [(layout, cfg, S, out, tm)
              for layout, cfgs in (("nk", TILED), ("kn", KN_TILED))
              for cfg in cfgs if cfg[:2] in ((256, 128), (256, 256))
              for S, out, tm in ((2, "f32", 3), (5, "bf16", 3), (8, "f16", 2), (8, "f32", 3))]


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="no GPU")
@pytest.mark.parametrize("case", SPLIT_FAST,
                         ids=lambda c: f"{c[0]}:tiled," + ",".join(map(str, c[1])) + f"-S{c[2]}-{c[3]}-tm{c[4]}")
def test_tiled_split_fastest_exact(hip_lib, case):
    layout, cfg, S, out, tm = case
    bm, bn = cfg[0], cfg[1]
    M, N, kps = tm * bm, 2 * bn + 40, 96
    K = (S - 1) * kps + 64
    dtype = "bf16"
    plan = _plan_text("tiled", cfg)
    text = hip_lib.describe_planned(plan, M, N, K, kps, S, inputs.DTYPES[dtype], layout=layout)
    print(f"case {layout} {dtype}->{out} M{M} N{N} K{K} kps{kps} S{S}: {text}", flush=True)
    assert f"bm{bm} bn{bn}" in text and text.endswith("splitfast"), text
    stored = (lambda t: t) if layout == "nk" else (lambda t: t.T.contiguous())
    dev = torch.device("cuda:0")
    ea, eb = inputs.exact_operands(M, N, K, dtype, seed=bm + bn + S + tm)
    ea64 = oracle.decode(inputs.stored_bits(ea), dtype)
    eb64 = oracle.decode(inputs.stored_bits(eb), dtype)
    EP, _, _ = oracle.splitk_partials(ea64, eb64, kps, S)
    EC = oracle.encode(EP.sum(axis=0), out).ravel()
    pbuf = inputs.guarded_buffer(S * M * N, "nan").to(dev)
    cbuf = inputs.guarded_buffer(M * N, "nan", dtype=out).to(dev)
    hip_lib.gemm_planned(plan, ea.to(dev), stored(eb).to(dev), pbuf[: S * M * N].view(S, M, N), kps, S,
                         C=cbuf[: M * N].view(M, N), layout=layout)
    torch.cuda.synchronize()
    p, c = pbuf.cpu().numpy(), inputs.stored_bits(cbuf.cpu())
    guard = np.float32(inputs.GUARD_VALUE).view(np.uint32)
    assert np.all(p[S * M * N:].view(np.uint32) == guard)
    np.testing.assert_array_equal(p[: S * M * N].astype(np.float64), EP.reshape(-1))
    np.testing.assert_array_equal(c[: M * N], EC)
    guard_c = inputs.stored_bits(inputs.guarded_buffer(0, "nan", dtype=out))
    assert np.all(c[M * N:] == guard_c)


# Persistent configurations with four or five tiles per workgroup (8 x 17
# tiles x 8 splits = 1088 on 256 workgroups), splits of two chunks (the
# second half empty for 16-bit inputs, so it is loaded through the zero
# piece and the re-read pieces), a 40-column last tile and a one-chunk last
# split; and 256x256 tiles at a split length of 10 and 16 chunks; both B
# layouts (with B as [K,N] the empty half of a two-chunk split re-reads the
# first half of its k-rows).  Exact-arithmetic inputs: every partial and the
# sum match the binary64 reference bit for bit.
PERSISTENT_MANY = ([("nk", c, "bf16", 96) for c in TILED_PT] +
                   [("nk", TILED_PT[0], "f16", 96), ("nk", TILED_PT[0], "f32", 96),
                    ("nk", TILED_PT[0], "bf16", 608), ("nk", TILED_PT[0], "bf16", 1024)] +
                   [("kn", c, dt, 96) for c in KN_TILED_PT for dt in ("bf16", "f16", "f32")] +
                   [("kn", KN_TILED_PT[0], "bf16", 608), ("kn", KN_TILED_PT[0], "bf16", 1024)])


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="no GPU")
@pytest.mark.parametrize("case", PERSISTENT_MANY,
                         ids=lambda c: f"{c[0]}:tiledp," + ",".join(map(str, c[1])) + f"-{c[2]}-kps{c[3]}")
def test_persistent_many_tiles_exact(hip_lib, case):
    layout, cfg, dtype, kps = case
    bm, bn = cfg[0], cfg[1]
    M, N, S = 2048, 16 * 256 + 40, 8
    K = (S - 1) * kps + 64
    plan = _plan_text("tiledp", cfg)
    text = hip_lib.describe_planned(plan, M, N, K, kps, S, inputs.DTYPES[dtype], layout=layout)
    print(f"case {layout} {dtype} M{M} N{N} K{K} kps{kps} S{S}: {text}", flush=True)
    assert text.endswith("grid256 persistent"), text
    stored = (lambda t: t) if layout == "nk" else (lambda t: t.T.contiguous())
    dev = torch.device("cuda:0")
    ea, eb = inputs.exact_operands(M, N, K, dtype, seed=bm + bn + kps)
    ea64 = oracle.decode(inputs.stored_bits(ea), dtype)
    eb64 = oracle.decode(inputs.stored_bits(eb), dtype)
    EP, _, _ = oracle.splitk_partials(ea64, eb64, kps, S)
    EC = EP.sum(axis=0)
    guard = np.float32(inputs.GUARD_VALUE).view(np.uint32)
    for poison in ("nan", "seven"):
        pbuf = inputs.guarded_buffer(S * M * N, poison).to(dev)
        cbuf = inputs.guarded_buffer(M * N, poison).to(dev)
        hip_lib.gemm_planned(plan, ea.to(dev), stored(eb).to(dev), pbuf[: S * M * N].view(S, M, N), kps, S,
                             C=cbuf[: M * N].view(M, N), layout=layout)
        torch.cuda.synchronize()
        p, c = pbuf.cpu().numpy(), cbuf.cpu().numpy()
        assert np.all(p[S * M * N:].view(np.uint32) == guard)
        assert np.all(c[M * N:].view(np.uint32) == guard)
        np.testing.assert_array_equal(p[: S * M * N].astype(np.float64), EP.reshape(-1))
        np.testing.assert_array_equal(c[: M * N].astype(np.float64), EC.reshape(-1))
