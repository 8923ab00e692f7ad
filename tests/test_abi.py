"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and rejects invalid arguments before touching the device."""
from __future__ import annotations

import ctypes
import glob
import os
import re
import subprocess

import pytest

import fp32_sgemm_02_amd as sg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions() -> set[str]:
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    declared = declared_functions()
    assert {"sgemm", "sgemm_ex", "sgemm_status_string", "sgemm_version"} <= declared
    out = subprocess.run(["nm", "-D", "--defined-only", sg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = declared - exported
    assert not missing, f"declared but not exported: {missing}"
    lib = ctypes.CDLL(sg.LIB_PATH)
    for name in declared:
        getattr(lib, name)


def test_version_and_tables():
    assert sg.version() == 500
    for v in (sg.VARIANT_MFMA, sg.VARIANT_VALU, sg.VARIANT_SKINNY):
        n = sg.tile_count(v)
        assert n > 0
        for t in range(n):
            d = sg.tile_info(v, t)
            assert d["bm"] > 0 and d["bn"] > 0 and d["threads"] % 64 == 0
            assert d["lds_bytes"] <= 160 * 1024
    assert sg.tile_count(0) == 0 and sg.tile_count(99) == 0
    with pytest.raises(sg.SgemmError):
        sg.tile_info(sg.VARIANT_MFMA, 999)


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, 4, 4, 4), -1),
    ((4, -1, 4, 4, 4, 4), -2),
    ((4, 4, -1, 4, 4, 4), -3),
    ((4, 4, 8, 7, 4, 4), -6),     # lda < K
    ((4, 8, 4, 4, 7, 8), -8),     # ldb < N
    ((4, 8, 4, 4, 8, 7), -11),    # ldc < N
    ((4, 4, 0, 0, 4, 4), -6),     # lda < max(1, K) with K = 0
])
def test_invalid_arguments_rejected_before_launch(args, code):
    M, N, K, lda, ldb, ldc = args
    fake = 0x1000   # never dereferenced: validation fails first
    assert sg.sgemm(M, N, K, 1.0, fake, lda, fake, ldb, 0.0, fake, ldc) == code
    assert sg.status_string(code).startswith(f"invalid argument {-code}")


def test_null_and_misaligned_pointers_rejected():
    good = 0x10000
    assert sg.sgemm(4, 4, 4, 1.0, None, 4, good, 4, 0.0, good, 4) == -5
    assert sg.sgemm(4, 4, 4, 1.0, good, 4, None, 4, 0.0, good, 4) == -7
    assert sg.sgemm(4, 4, 4, 1.0, good, 4, good, 4, 0.0, None, 4) == -10
    assert sg.sgemm(4, 4, 4, 1.0, good + 2, 4, good, 4, 0.0, good, 4) == -5
    assert sg.sgemm(4, 4, 4, 1.0, good, 4, good + 1, 4, 0.0, good, 4) == -7
    assert sg.sgemm(4, 4, 4, 1.0, good, 4, good, 4, 0.0, good + 3, 4) == -10


def test_empty_products_are_no_ops_without_device():
    # M == 0 or N == 0 return before any device call, even with null pointers
    assert sg.sgemm(0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4) == 0
    assert sg.sgemm(4, 0, 4, 1.0, None, 4, None, 1, 0.0, None, 1) == 0
    # alpha == 0 with beta == 1 leaves C untouched: nothing is launched
    assert sg.sgemm(4, 4, 4, 0.0, None, 4, None, 4, 1.0, 0x10000, 4) == 0
    # K == 0 with beta == 1 likewise
    assert sg.sgemm(4, 4, 0, 1.0, None, 1, None, 4, 1.0, 0x10000, 4) == 0


def test_bad_configuration():
    good = 0x10000
    cfg = sg.SgemmConfig(99, -1, 0, 0)
    assert sg.sgemm_ex(4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4, None, cfg) == -13
    cfg = sg.SgemmConfig(sg.VARIANT_MFMA, 999, 0, 0)
    assert sg.sgemm_ex(64, 64, 4, 1.0, good, 4, good, 64, 0.0, good, 64, None, cfg) == -13
    # the skinny family does not apply to a 64 x 64 product
    cfg = sg.SgemmConfig(sg.VARIANT_SKINNY, -1, 0, 0)
    assert sg.sgemm_ex(64, 64, 4, 1.0, good, 4, good, 64, 0.0, good, 64, None, cfg) == -13
    # a few-columns tile cannot serve a few-rows shape with many columns
    kind1 = [t for t in range(sg.tile_count(sg.VARIANT_SKINNY))
             if sg.tile_info(sg.VARIANT_SKINNY, t)["tm"] == 1][-1]
    cfg = sg.SgemmConfig(sg.VARIANT_SKINNY, kind1, 0, 0)
    assert sg.sgemm_ex(8, 64, 4, 1.0, good, 4, good, 64, 0.0, good, 64, None, cfg) == -13


def test_transposed_entry_point_validation():
    """sgemm_op checks its trans flags and the transposed leading dimensions
    before touching the device, and refuses what no kernel serves."""
    good = 0x10000
    op = sg.sgemm_op
    assert op(2, 0, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -21
    assert op(0, -1, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -22
    # A stored K x M: lda must cover M
    assert op(1, 0, 8, 4, 2, 1.0, good, 4, good, 4, 0.0, good, 4) == -6
    # B stored N x K: ldb must cover K
    assert op(0, 1, 4, 8, 6, 1.0, good, 6, good, 4, 0.0, good, 8) == -8
    assert op(0, 1, -1, 8, 6, 1.0, good, 6, good, 6, 0.0, good, 8) == -1
    # transposed A: only the tiles flagged for it, and those serve nothing else
    ta = [t for t in range(sg.tile_count(sg.VARIANT_MFMA))
          if sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_TRANS_A]
    assert ta, "no tile serves transposed A"
    for t in range(sg.tile_count(sg.VARIANT_MFMA)):
        cfg = sg.SgemmConfig(sg.VARIANT_MFMA, t, 0, 0)
        for trans_a in (0, 1):
            if (t in ta) != bool(trans_a):
                assert op(trans_a, 0, 256, 256, 64, 1.0, good, 256, good, 256, 0.0, good, 256,
                          None, cfg) == -13, (t, trans_a)
    for variant in (sg.VARIANT_VALU, sg.VARIANT_SKINNY):
        cfg = sg.SgemmConfig(variant, -1, 0, 0)
        assert op(1, 0, 64, 64, 64, 1.0, good, 64, good, 64, 0.0, good, 64, None, cfg) == -13
    # the few-columns skinny kernel does not read A transposed
    kind1 = [t for t in range(sg.tile_count(sg.VARIANT_SKINNY))
             if sg.tile_info(sg.VARIANT_SKINNY, t)["tm"] == 1][-1]
    cfg = sg.SgemmConfig(sg.VARIANT_SKINNY, kind1, 0, 0)
    assert op(1, 0, 64, 8, 64, 1.0, good, 64, good, 8, 0.0, good, 8, None, cfg) == -13
    # transposed B: the MFMA tiles flagged for it and the skinny family (on
    # skinny shapes); never the VALU family
    for variant in (sg.VARIANT_VALU, sg.VARIANT_SKINNY):
        cfg = sg.SgemmConfig(variant, -1, 0, 0)
        assert op(0, 1, 64, 64, 64, 1.0, good, 64, good, 64, 0.0, good, 64, None, cfg) == -13
    tb = [t for t in range(sg.tile_count(sg.VARIANT_MFMA))
          if sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_TRANS_B]
    assert tb, "no tile serves transposed B"
    for t in range(sg.tile_count(sg.VARIANT_MFMA)):
        if t in tb:
            continue
        cfg = sg.SgemmConfig(sg.VARIANT_MFMA, t, 0, 0)
        assert op(0, 1, 256, 256, 64, 1.0, good, 64, good, 64, 0.0, good, 256, None, cfg) == -13
    # quick returns need no kernel: alpha == 0 with beta == 1, empty shapes
    assert op(1, 1, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, good, 4) == 0
    assert op(1, 1, 0, 4, 4, 1.0, None, 1, None, 4, 0.0, None, 4) == 0


def whole_tiles():
    return [t for t in range(sg.tile_count(sg.VARIANT_MFMA))
            if sg.tile_info(sg.VARIANT_MFMA, t)["flags"] & sg.TILE_WHOLE]


def test_whole_tiles_rejected_where_they_cannot_run():
    """Whole-tile (direct-load) configurations refuse, before any launch,
    shapes that are not made of whole tiles, unaligned operands and scalar I/O."""
    assert whole_tiles(), "no whole-tile MFMA configuration compiled"
    good = 0x10000
    for t in whole_tiles():
        d = sg.tile_info(sg.VARIANT_MFMA, t)
        bm, bn, bk = d["bm"], d["bn"], d["bk"]
        for (M, N, K) in ((bm + 1, bn, 4 * bk), (bm, bn + 4, 4 * bk), (bm, bn, 4 * bk + 4),
                          (2 * bm - 16, bn, bk), (bm, bn, bk // 2)):
            cfg = sg.SgemmConfig(sg.VARIANT_MFMA, t, 0, 0)
            assert sg.sgemm_ex(M, N, K, 1.0, good, K, good, N, 0.0, good, N, None, cfg) == -13
        M, N, K = 2 * bm, bn, 4 * bk
        cfg = sg.SgemmConfig(sg.VARIANT_MFMA, t, sg.FLAG_SCALAR_IO, 0)
        assert sg.sgemm_ex(M, N, K, 1.0, good, K, good, N, 0.0, good, N, None, cfg) == -13
        cfg = sg.SgemmConfig(sg.VARIANT_MFMA, t, 0, 0)
        assert sg.sgemm_ex(M, N, K, 1.0, good + 4, K, good, N, 0.0, good, N, None, cfg) == -13
        assert sg.sgemm_ex(M, N, K, 1.0, good, K + 2, good, N, 0.0, good, N, None, cfg) == -13


def test_automatic_selection_never_picks_an_inapplicable_whole_tile():
    for (M, N, K) in ((4096, 4096, 4096), (8192, 8192, 8192), (8192, 14336, 4096)):
        for a in (0x10000, 0x10004):
            cfg = sg.select(M, N, K, a, K, 0x20000, N, 0x30000, N)
            d = sg.tile_info(cfg.variant, cfg.tile)
            if d["flags"] & sg.TILE_WHOLE:
                assert a % 16 == 0 and M % d["bm"] == 0 and N % d["bn"] == 0
        # one row more: a whole tile only for the main part, with the row split off
        cfg, rows, cols = sg.plan(M + 1, N, K, 0x10000, K, 0x20000, N, 0x30000, N)
        d = sg.tile_info(cfg.variant, cfg.tile)
        if d["flags"] & sg.TILE_WHOLE:
            assert rows == 1 and (M + 1 - rows) % d["bm"] == 0 and (N - cols) % d["bn"] == 0
    # untuned large shapes, whole or ragged, get a direct-load tile; a ragged
    # one never a whole-tile one
    cfg = sg.select(6144, 6144, 6144, 0x10000, 6144, 0x20000, 6144, 0x30000, 6144)
    assert sg.tile_info(cfg.variant, cfg.tile)["flags"] & sg.TILE_DIRECT
    cfg = sg.select(6143, 6144, 6143, 0x10000, 6143, 0x20000, 6144, 0x30000, 6144)
    d = sg.tile_info(cfg.variant, cfg.tile)
    assert d["flags"] & sg.TILE_DIRECT and not d["flags"] & sg.TILE_WHOLE


def test_edge_strip_plan():
    """The automatic plan hands at most 16 edge rows / columns to the skinny
    family, only when they would cost an extra round of workgroups, and the
    main part then divides into the chosen tile's rows / columns."""
    a, b, c = 0x10000, 0x20000, 0x30000
    cfg, rows, cols = sg.plan(4097, 1000, 3001, a, 3001, b, 1000, c, 1000)
    assert (rows, cols) == (1, 0)
    d = sg.tile_info(cfg.variant, cfg.tile)
    assert cfg.variant == sg.VARIANT_MFMA and 4096 % d["bm"] == 0
    assert d["flags"] & sg.TILE_DIRECT
    for (M, N, K) in ((4096, 4096, 4096), (300, 257, 129), (1000, 1000, 1000), (4200, 4100, 512),
                      (2049, 2048, 2048), (2048, 2051, 700), (8193, 8200, 100), (20, 5000, 64)):
        cfg, rows, cols = sg.plan(M, N, K, a, K, b, N, c, N)
        d = sg.tile_info(cfg.variant, cfg.tile)
        assert 0 <= rows <= 16 and 0 <= cols <= 16
        if rows:
            assert (M - rows) % d["bm"] == 0 and M - rows >= d["bm"]
        if cols:
            assert (N - cols) % d["bn"] == 0 and N - cols >= d["bn"]
        if (M, N, K) == (4096, 4096, 4096):
            assert (rows, cols) == (0, 0)
        if cfg.variant == sg.VARIANT_SKINNY:
            assert (rows, cols) == (0, 0)


def test_automatic_selection():
    assert sg.select(4096, 4096, 4096).variant == sg.VARIANT_MFMA
    assert sg.select(1, 4096, 4096).variant == sg.VARIANT_SKINNY
    assert sg.select(4096, 1, 4096).variant == sg.VARIANT_SKINNY
    assert sg.select(16, 14336, 4096).variant == sg.VARIANT_SKINNY
    # lda = 33 rules out 16-byte A rows: a general tile runs its 4-byte path,
    # a direct-load, skinny or small-product tile picks the width per operand
    cfg = sg.select(777, 777, 33, 0x10000, 33)
    d = sg.tile_info(cfg.variant, cfg.tile)
    assert (cfg.flags & sg.FLAG_SCALAR_IO or d["flags"] & sg.TILE_DIRECT or
            cfg.variant == sg.VARIANT_SMALL)
    assert sg.select(256, 256, 256, 0x10000, 256, 0x20000, 256, 0x30000, 256).flags == 0


def test_lone_workgroup_tiles_give_way_to_k_groups():
    """Where the 8-wave 128 x 128 tile would fill exactly one round of
    workgroups (one per CU), the plan takes a tile with k-groups (measured
    3.4-6.5 % faster there); from two rounds on it keeps the 128 x 128 tile."""
    a, b, c = 0x10000, 0x20000, 0x30000

    def kgroups(M, N, K):
        cfg, rows, cols = sg.plan(M, N, K, a, K, b, N, c, N)
        d = sg.tile_info(cfg.variant, cfg.tile)
        per_group = (d["bm"] // d["wm"]) * (d["bn"] // d["wn"])
        return cfg.variant, d["threads"] // 64 // per_group, (d["bm"], d["bn"])

    for shape in ((4096, 1024, 4096), (2048, 2048, 4096), (1024, 4096, 4096), (4096, 1000, 1000)):
        variant, kg, _ = kgroups(*shape)
        assert variant == sg.VARIANT_MFMA and kg == 2, shape
    variant, kg, tile = kgroups(4096, 2048, 4096)
    assert (variant, kg, tile) == (sg.VARIANT_MFMA, 1, (128, 128))
    # the ragged workload: the main part on a k-group tile, the last row split off
    cfg, rows, cols = sg.plan(4097, 1000, 3001, a, 3001, b, 1000, c, 1000)
    d = sg.tile_info(cfg.variant, cfg.tile)
    assert rows == 1 and d["threads"] // 64 > (d["bm"] // d["wm"]) * (d["bn"] // d["wn"])


def test_small_product_selection():
    """Fewer than 256 tiles of 64 x 64 (over the batch), at most 1.5 GFLOP,
    A untransposed: the small-product family, 16 x 64 blocks where B's rows
    take 16-byte loads and such blocks are many, 16 x 16 blocks otherwise,
    k-groups for long K; otherwise (or M / N <= 16) another family."""
    a, b, c = 0x10000, 0x20000, 0x30000

    def pick(M, N, K, **kw):
        cfg = sg.select(M, N, K, a, K, b, N, c, N, **kw)
        return cfg.variant, cfg.tile

    assert pick(256, 256, 256) == (sg.VARIANT_SMALL, 0)    # few 16 x 64 blocks: 16 x 16
    assert pick(384, 384, 384) == (sg.VARIANT_SMALL, 2)
    assert pick(512, 512, 512) == (sg.VARIANT_SMALL, 2)
    assert pick(777, 777, 33) == (sg.VARIANT_SMALL, 1)     # N % 4 != 0: 16 x 16 blocks
    assert pick(256, 256, 4096) == (sg.VARIANT_SMALL, 5)   # long K: 8 k-groups
    assert pick(512, 512, 2048) == (sg.VARIANT_SMALL, 2)
    assert pick(64, 64, 64) == (sg.VARIANT_SMALL, 1)       # a few k-steps, few blocks
    assert pick(1024, 1024, 1024)[0] == sg.VARIANT_MFMA     # 256 tiles of 64 x 64
    assert pick(1000, 1000, 64) == (sg.VARIANT_SMALL, 7)    # ... with K <= 64: no k-groups
    assert pick(768, 768, 65536)[0] == sg.VARIANT_MFMA      # 77 GFLOP: stream-K
    # narrow products (M or N <= 200) with long K: the family whatever their
    # flops, while C covers less than 200 tiles of 64 x 64 in area
    assert pick(64, 4096, 4096) == (sg.VARIANT_SMALL, 6)
    assert pick(4096, 48, 8192) == (sg.VARIANT_SMALL, 6)
    assert pick(32, 14336, 4096) == (sg.VARIANT_SMALL, 3)
    assert pick(64, 14336, 4096)[0] == sg.VARIANT_MFMA
    assert pick(3000, 100, 3000) == (sg.VARIANT_SMALL, 2)
    assert pick(16, 4096, 4096)[0] == sg.VARIANT_SKINNY
    assert pick(256, 256, 256, trans_a=True)[0] == sg.VARIANT_MFMA
    assert pick(384, 384, 384, trans_b=True) == (sg.VARIANT_SMALL, 2)


def test_cblas_entry_point_validation():
    """sgemm_cblas takes cblas_sgemm's enumerations and names the caller's
    arguments in its status codes, also for column-major calls (which run as
    the row-major product with the operands swapped)."""
    good = 0x10000
    cb = sg.sgemm_cblas
    RM, CM, NT, T, CT = 101, 102, 111, 112, 113
    assert cb(100, NT, NT, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -23
    assert cb(RM, 0, NT, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -21
    assert cb(CM, NT, 1, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -22
    for order in (RM, CM):
        assert cb(order, NT, NT, -1, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -1
        assert cb(order, NT, NT, 4, -1, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -2
        assert cb(order, NT, NT, 4, 4, -1, 1.0, good, 4, good, 4, 0.0, good, 4) == -3
        assert cb(order, T, CT, 4, 4, 4, 1.0, None, 4, good, 4, 0.0, good, 4) == -5
        assert cb(order, NT, NT, 4, 4, 4, 1.0, good, 4, None, 4, 0.0, good, 4) == -7
        assert cb(order, NT, NT, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, None, 4) == -10
    # column-major A (M x K, no transpose) needs lda >= M; row-major needs lda >= K
    assert cb(CM, NT, NT, 8, 4, 2, 1.0, good, 4, good, 8, 0.0, good, 8) == -6
    assert cb(CM, NT, NT, 8, 4, 2, 1.0, good, 8, good, 1, 0.0, good, 8) == -8
    assert cb(CM, NT, NT, 8, 4, 2, 1.0, good, 8, good, 2, 0.0, good, 4) == -11
    assert cb(CM, T, NT, 8, 4, 2, 1.0, good, 1, good, 2, 0.0, good, 8) == -6
    assert cb(CM, NT, T, 8, 4, 2, 1.0, good, 8, good, 2, 0.0, good, 8) == -8
    # quick returns need no kernel
    for order in (RM, CM):
        assert cb(order, T, T, 0, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == 0
        assert cb(order, NT, T, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, good, 4) == 0


def test_op_plan_covers_transpositions():
    """The automatic plan of a transposed product names a tile that serves
    that transposition: the skinny family on skinny shapes (few rows: any
    transposition; few columns: A untransposed), the small-product family
    (B either way, A untransposed) on products of few 64 x 64 tiles, else an
    MFMA tile flagged for it; edge strips only with A untransposed."""
    for ta, tb in ((0, 1), (1, 0), (1, 1)):
        for M, N, K in ((4096, 4096, 4096), (4097, 1000, 3001), (2049, 2048, 64), (37, 45, 5),
                        (1, 4096, 4096), (16, 14336, 4096), (4096, 1, 4096)):
            cfg, rows, cols = sg.plan(M, N, K, 0x10000, None, 0x10000, None, 0x10000, None,
                                      trans_a=ta, trans_b=tb)
            lab = (ta, tb, M, N, K)
            if M <= 16 or (N <= 16 and not ta):
                assert cfg.variant == sg.VARIANT_SKINNY, lab
                continue
            if cfg.variant == sg.VARIANT_SMALL:
                assert not ta and (M // 64 + 1) * (N // 64 + 1) < 300, lab
                assert sg.tile_info(sg.VARIANT_SMALL, cfg.tile)["flags"] & sg.TILE_TRANS_B, lab
                continue
            assert cfg.variant == sg.VARIANT_MFMA, lab
            f = sg.tile_info(sg.VARIANT_MFMA, cfg.tile)["flags"]
            assert bool(f & sg.TILE_TRANS_A) == bool(ta), lab
            if tb:
                assert f & sg.TILE_TRANS_B, lab
            if ta:
                assert (rows, cols) == (0, 0), lab
    a, b = sg.plan(64, 64, 64, trans_a=False), sg.plan(64, 64, 64)
    assert (a[0].variant, a[0].tile, a[1:]) == (b[0].variant, b[0].tile, b[1:])
    out = sg.SgemmConfig()
    lib = sg._load()
    assert lib.sgemm_op_plan(2, 0, 4, 4, 4, None, 4, None, 4, None, 4, ctypes.byref(out),
                             None, None) == -21
    assert lib.sgemm_op_plan(0, 5, 4, 4, 4, None, 4, None, 4, None, 4, ctypes.byref(out),
                             None, None) == -22


def test_one_row_with_b_transposed_plans_no_split():
    """One row of C with B stored transposed (x W^T) and no bias runs as the
    one-column product (C^T = W x^T), which splits nothing: its plan reports
    one K slice, where the same row with B untransposed is split over K.  When
    the one-column kernel cannot take it (x not 16-byte aligned), the few-rows
    kernel runs it and the plan reports that kernel's slices."""
    nt, _, _ = sg.plan(1, 4096, 4096, 0x10000, None, 0x20000, None, 0x30000, None, trans_b=True)
    nn, _, _ = sg.plan(1, 4096, 4096, 0x10000, None, 0x20000, None, 0x30000, None)
    assert nt.variant == nn.variant == sg.VARIANT_SKINNY
    assert nt.group_m == 1, nt.group_m
    assert nn.group_m > 1, nn.group_m
    # x 4 bytes past a 16-byte boundary: the few-rows kernel and its split
    rows, _, _ = sg.plan(1, 4096, 4096, 0x10004, None, 0x20000, None, 0x30000, None,
                         trans_b=True)
    assert rows.variant == sg.VARIANT_SKINNY and rows.group_m > 1, (rows.tile, rows.group_m)


def test_epilogue_entry_point_validation():
    """sgemm_epilogue: act codes, bias alignment, and the quick returns that
    no longer apply when an epilogue is asked for are checked on the host."""
    good = 0x10000
    ep = sg.sgemm_epilogue
    assert ep(0, 0, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4, good, 5) == -25
    assert ep(0, 0, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4, good, -1) == -25
    assert ep(0, 0, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4, good + 2, 1) == -24
    assert ep(2, 0, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4, good, 1) == -21
    assert ep(0, 0, -1, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4, good, 1) == -1
    assert ep(0, 0, 4, 4, 4, 1.0, None, 4, good, 4, 0.0, good, 4, good, 1) == -5
    # empty C: nothing to do, whatever the epilogue
    assert ep(0, 0, 0, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4, good, 1) == 0
    # no bias and no activation is sgemm_op
    assert ep(0, 0, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, good, 4, None, 0) == 0


def test_batched_entry_point_validation():
    """sgemm_strided_batched: batch, stride and overlap checks on the host."""
    good = 0x10000
    bt = sg.sgemm_strided_batched
    args = lambda **kw: dict(dict(ta=0, tb=0, M=4, N=4, K=4, alpha=1.0, A=good, lda=4, sa=16,
                                  B=good, ldb=4, sb=16, beta=0.0, C=good, ldc=4, sc=16, batch=3),
                             **kw)
    call = lambda d: bt(d["ta"], d["tb"], d["M"], d["N"], d["K"], d["alpha"], d["A"], d["lda"],
                        d["sa"], d["B"], d["ldb"], d["sb"], d["beta"], d["C"], d["ldc"], d["sc"],
                        d["batch"])
    assert call(args(batch=-1)) == -29
    assert call(args(sa=-16)) == -26
    assert call(args(sb=-1)) == -27
    assert call(args(sc=15)) == -28          # C_1 would overlap C_0
    assert call(args(sc=0)) == -28
    assert call(args(tb=3)) == -22
    assert call(args(M=-2)) == -1
    assert call(args(ldb=3)) == -8
    # shared operands (stride 0) are allowed; batch 0 and batch 1 need no C stride
    assert call(args(batch=0, sc=0)) == 0
    assert call(args(M=0, sc=0)) == 0
    assert call(args(alpha=0.0, beta=1.0, A=None, B=None, sa=0, sb=0)) == 0


def test_mixed_entry_point_validation():
    """sgemm_mixed: dtype and argument checks on the host; the 16-bit tile
    tables are described."""
    good = 0x10000
    mx = sg.sgemm_mixed
    assert mx(0, 0, 1, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -30
    assert mx(3, 0, 1, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -30
    assert mx(sg.DTYPE_BF16, 2, 1, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -21
    assert mx(sg.DTYPE_F16, 0, 1, -1, 4, 4, 1.0, good, 4, good, 4, 0.0, good, 4) == -1
    assert mx(sg.DTYPE_F16, 0, 1, 4, 4, 4, 1.0, good, 3, good, 4, 0.0, good, 4) == -6
    assert mx(sg.DTYPE_F16, 0, 1, 4, 4, 4, 1.0, good + 1, 4, good, 4, 0.0, good, 4) == -5
    assert mx(sg.DTYPE_BF16, 0, 1, 4, 4, 4, 1.0, good, 4, good, 4, 0.0, good + 2, 4) == -10
    assert mx(sg.DTYPE_BF16, 0, 1, 0, 4, 4, 1.0, None, 4, None, 4, 0.0, None, 4) == 0
    assert mx(sg.DTYPE_BF16, 0, 1, 4, 4, 4, 0.0, None, 4, None, 4, 1.0, good, 4) == 0
    # the matrix-core tiles need A untransposed, B transposed, even K
    cfg = sg.SgemmConfig(sg.VARIANT_MFMA16, 0, 0, 0)
    assert mx(sg.DTYPE_BF16, 0, 0, 64, 64, 64, 1.0, good, 64, good, 64, 0.0, good, 64,
              None, cfg) == -13
    assert mx(sg.DTYPE_BF16, 0, 1, 64, 64, 63, 1.0, good, 63, good, 63, 0.0, good, 64,
              None, cfg) == -13
    assert sg.tile_count(sg.VARIANT_MFMA16) > 0 and sg.tile_count(sg.VARIANT_GENERIC16) == 1
    for t in range(sg.tile_count(sg.VARIANT_MFMA16)):
        d = sg.tile_info(sg.VARIANT_MFMA16, t)
        assert d["flags"] & sg.TILE_TRANS_B and d["bk"] % 2 == 0
    # fp32 entry points refuse the 16-bit families
    cfg = sg.SgemmConfig(sg.VARIANT_MFMA16, 0, 0, 0)
    assert sg.sgemm_ex(64, 64, 64, 1.0, good, 64, good, 64, 0.0, good, 64, None, cfg) == -13


# The shapes of the named workloads: (M, N, K).  Square sweep 128 .. 8192.
NAMED_SHAPES = ([(256, 256, 256), (4096, 4096, 4096), (4097, 1000, 3001), (1, 4096, 4096),
                 (4096, 1, 4096), (777, 777, 33), (8192, 14336, 4096), (8192, 4096, 14336),
                 (16, 14336, 4096)] + [(n, n, n) for n in (128, 256, 512, 1024, 2048, 4096, 8192)])
STATIC_SCRATCH_BYTES = 16 << 20   # sgemm_op_ex_noalloc's array, after its counters


def plan_partial_bytes(M, N, K, a=0x10000, b=0x20000, c=0x30000, lda=None, ldb=None, ldc=None):
    """(configuration, partial-sum bytes) of one part of an automatic plan:
    a stream-K launch keeps two tile accumulators per workgroup, a few-rows
    skinny launch split into S K-slices keeps S x M x N floats."""
    cfg, rows, cols = sg.plan(M, N, K, a, lda or K, b, ldb or N, c, ldc or N)
    d = sg.tile_info(cfg.variant, cfg.tile)
    if cfg.flags & sg.FLAG_STREAMK:
        return cfg, rows, cols, 2 * 256 * 4 * d["bm"] * d["bn"]
    if cfg.variant == sg.VARIANT_SKINNY and d["tm"] == 0 and cfg.group_m > 1:
        return cfg, rows, cols, cfg.group_m * M * N * 4
    return cfg, rows, cols, 0


def test_named_workload_plans_take_no_stream_k_and_fit_the_static_scratch():
    """Which automatic plans of the named workloads keep partial sums in
    device memory: none is stream-K (64-128 MiB); the few-rows products
    whose strips leave CUs idle are split over K (1 x 4096 x 4096, the
    16-row decode shape, the one-row edge strip of 4097 x 1000 x 3001), and
    their partial sums fit the static scratch of the entry point that
    allocates nothing, so that entry point runs the same plans."""
    split = {}
    for M, N, K in NAMED_SHAPES:
        cfg, rows, cols, ws = plan_partial_bytes(M, N, K)
        assert not cfg.flags & sg.FLAG_STREAMK, (M, N, K)
        assert ws <= STATIC_SCRATCH_BYTES, (M, N, K, ws)
        if ws:
            split[(M, N, K)] = ws
        if rows:   # the edge strip below the main part: its own plan
            _, _, _, ws_rows = plan_partial_bytes(rows, N, K, a=0x10000 + 4 * (M - rows) * K)
            assert ws_rows <= STATIC_SCRATCH_BYTES
            if ws_rows:
                split[(rows, N, K, "edge rows")] = ws_rows
    assert set(split) == {(1, 4096, 4096), (16, 14336, 4096), (1, 1000, 3001, "edge rows")}, split
    assert split[(1, 4096, 4096)] <= 1 << 20
