"""Generate the tile-kernel instantiations and their registry.

The candidate family is a grid over the knobs a matmul autotuner searches:
block shape BM x BN, reduction depth BK, waves per workgroup, pipeline stages,
operand storage (layout), the width of the operands' vector loads (which the
key's stride factors decide), and split-K.  Each point is one instantiation
of tile_kernel.h's template, compiled ahead of time for gfx950.

Writes, into the given output directory:
  tiles_<n>.hip          launcher definitions, a few per file so the build
                         can compile them in parallel
  tile_registry.inc      one initializer per instantiation, read by
                         candidates.cpp (order = registration order)
"""
import os
import sys

TRAITS = {"f32": "TraitsF32", "f16": "TraitsF16", "bf16": "TraitsBF16", "e4m3": "TraitsFP8"}
DT_CODE = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
CH = {"f32": 4, "f16": 8, "bf16": 8, "e4m3": 16}
E = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}
LAYOUT_CODE = {"NN": 0, "NT": 1, "TN": 2, "TT": 3}

# waves per workgroup -> (waves along M, waves along N) for a block shape
def wave_grid(BM, BN, waves):
    if waves == 4:
        return 2, 2
    if waves == 8:
        return (2, 4) if BN >= BM else (4, 2)
    if waves == 1:
        return 1, 1
    raise ValueError(waves)


def tile(dtype, layout, BM, BN, BK, waves, stages, va=None, vb=None, splitk=False, dma=False, xpose=False,
         m16=False, grid=None, wtn=128, half=False, wk=1):
    WM, WN = grid if grid else wave_grid(BM, BN, waves)
    if m16 and layout == "NN" and not xpose:  # tile_dma16n.h: wave tiles wtn (128 or 64) columns wide
        WN = BN // wtn
        WM = waves // WN
    full = CH[dtype]
    va = full if va is None else va
    vb = full if vb is None else vb
    assert not dma or (va == full and vb == full), "LDS-DMA copies whole 16-byte chunks"
    assert not m16 or (dma and (layout in ("NT", "NN") or xpose) and E[dtype] == 2), "16x16x32 blocks: 16-bit, A K-major"
    assert not half or (dma and not m16 and (layout == "NT" or xpose)), "half-split 32x32 blocks: K-major"
    assert wk == 1 or not (dma or splitk), "k-groups in register-staged tiles without a k-split"
    return dict(dtype=dtype, layout=layout, BM=BM, BN=BN, BK=BK, WM=WM, WN=WN, ST=stages, VA=va, VB=vb,
                splitk=splitk, dma=dma, xpose=xpose, m16=m16, half=half, WK=wk)


def dma_tile(dtype, layout, BM, BN, BK, waves, stages, splitk=False):
    """LDS-DMA variant (tile_dma.h): both operands copied straight into
    `stages` LDS buffers."""
    return tile(dtype, layout, BM, BN, BK, waves, stages, splitk=splitk, dma=True)


def xpose_tile(dtype, layout, BM, BN, BK, waves, stages, m16=False, grid=None):
    """Composite: the MN-major operand(s) transposed into the workspace, then
    the K-major (NT) LDS-DMA kernel."""
    assert layout != "NT"
    return tile(dtype, layout, BM, BN, BK, waves, stages, dma=True, xpose=True, m16=m16, grid=grid)


def m16_tile(dtype, BM, BN, BK, waves, stages, splitk=False, grid=None):
    """LDS-DMA NT tile built from 16x16x32 matrix-core blocks (tile_dma16.h)."""
    return tile(dtype, "NT", BM, BN, BK, waves, stages, splitk=splitk, dma=True, m16=True, grid=grid)


def nn16_tile(dtype, BM, BN, BK, waves, stages, splitk=False, wtn=128):
    """LDS-DMA NN tile built from 16x16x32 matrix-core blocks, B read
    MN-major and transposed in registers (tile_dma16n.h); wave tiles wtn
    columns wide (128: 16-byte reads of B, 64: 8-byte reads)."""
    return tile(dtype, "NN", BM, BN, BK, waves, stages, splitk=splitk, dma=True, m16=True, wtn=wtn)


def xpose_bits(t):
    """1: lhs transposed into the workspace, 2: rhs."""
    if not t["xpose"]:
        return 0
    return (1 if t["layout"][0] == "T" else 0) | (2 if t["layout"][1] == "N" else 0)


def lds_bytes(t):
    if t["dma"]:
        nbuf = t["ST"]
    else:
        nbuf = 1 if t["ST"] == 1 else 2
    tiles = nbuf * (t["BM"] + t["BN"]) * t["BK"] * E[t["dtype"]]
    wk = t.get("WK", 1)
    # k-groups: the other groups' fp32 sums pass through the same LDS
    return max(tiles, (wk - 1) * t["BM"] * t["BN"] * 4) if wk > 1 else tiles


# kernel family codes of the tile registry (candidates.cpp: TileFamily)
KF_REG, KF_DMA, KF_DMA16, KF_DMAH = 0, 1, 2, 3


def kernel_family(t):
    """Which tile kernel an instantiation uses: register-staged, LDS-DMA on
    32x32 blocks, LDS-DMA on 16x16 blocks, LDS-DMA with half-split k-steps."""
    if not t["dma"]:
        return KF_REG
    return KF_DMA16 if t["m16"] else KF_DMAH if t["half"] else KF_DMA


def name_of(t):
    kind = "splitk" if t["splitk"] else "tile"
    if t["dma"]:
        kind = ("xdma" if t["xpose"] else "dma") + ("16_" if t["m16"] else "h_" if t["half"] else "_") + kind
    v = ""
    full = CH[t["dtype"]]
    if t["VA"] != full or t["VB"] != full:
        v = "_va%dvb%d" % (t["VA"], t["VB"])
    w = "%dx%d" % (t["WM"], t["WN"]) + ("x%d" % t["WK"] if t.get("WK", 1) > 1 else "")
    return "%s_%s_%s_%dx%dx%d_w%s_s%d%s" % (kind, t["dtype"], t["layout"].lower(), t["BM"], t["BN"], t["BK"], w,
                                           t["ST"], v)


def reg_tile_fits(BM, BN, waves, stages):
    """Register-staged tiles that compile without scratch on gfx950: a third
    stage (a second set of staging registers) only for blocks up to 128x128,
    and 8 waves not on 256x256 blocks (their staging plus accumulators exceed
    the 256 VGPRs a wave gets at two waves per SIMD).  The LDS-DMA variants
    cover those shapes."""
    if stages == 3 and BM * BN > 128 * 128:
        return False
    if waves == 8 and BM * BN >= 256 * 256:
        return False
    return True


def family():
    out = []
    # bf16: the full grid for NN and NT (>= 24 shape/wave/stage combinations)
    for layout in ("NN", "NT"):
        for BM, BN in ((128, 128), (128, 256), (256, 128), (256, 256)):
            for waves in (4, 8):
                for BK in (32, 64):
                    for st in (1, 2, 3):
                        if reg_tile_fits(BM, BN, waves, st):
                            out.append(tile("bf16", layout, BM, BN, BK, waves, st))
        for BM, BN in ((64, 64), (64, 128), (128, 64)):
            out.append(tile("bf16", layout, BM, BN, 64, 4, 2))
        out.append(tile("bf16", layout, 128, 128, 64, 4, 2, va=1, vb=1))
        out.append(tile("bf16", layout, 64, 64, 64, 4, 2, va=1, vb=1))
        for BM, BN in ((64, 64), (128, 128)):
            out.append(tile("bf16", layout, BM, BN, 64, 4, 2, splitk=True))
            out.append(tile("bf16", layout, BM, BN, 64, 4, 2, va=1, vb=8, splitk=True))
    for layout in ("TN", "TT"):
        out.append(tile("bf16", layout, 128, 128, 64, 4, 2))
        out.append(tile("bf16", layout, 128, 128, 64, 4, 2, va=1, vb=1))
        out.append(tile("bf16", layout, 64, 64, 64, 4, 2, splitk=True))
    # f16: a smaller grid
    for layout in ("NN", "NT"):
        for BM, BN, waves in ((128, 128, 4), (256, 256, 4), (256, 128, 8)):
            out.append(tile("f16", layout, BM, BN, 64, waves, 2))
        out.append(tile("f16", layout, 64, 64, 64, 4, 2))
        out.append(tile("f16", layout, 128, 128, 64, 4, 2, va=1, vb=1))
        out.append(tile("f16", layout, 64, 64, 64, 4, 2, splitk=True))
        out.append(tile("f16", layout, 128, 128, 64, 4, 2, va=1, vb=8, splitk=True))
    for layout in ("TN", "TT"):
        out.append(tile("f16", layout, 128, 128, 64, 4, 2))
        out.append(tile("f16", layout, 128, 128, 64, 4, 2, va=1, vb=1))
    # fp8 e4m3
    for layout in ("NN", "NT"):
        for BM, BN in ((128, 128), (128, 256), (256, 128), (256, 256)):
            for waves in (4, 8):
                for BK, st in ((64, 2), (128, 2), (128, 3)):
                    if reg_tile_fits(BM, BN, waves, st):
                        out.append(tile("e4m3", layout, BM, BN, BK, waves, st))
        out.append(tile("e4m3", layout, 64, 64, 64, 4, 2))
        out.append(tile("e4m3", layout, 128, 128, 64, 4, 2, va=1, vb=1))
        out.append(tile("e4m3", layout, 64, 64, 64, 4, 2, splitk=True))
        out.append(tile("e4m3", layout, 128, 128, 128, 4, 2, splitk=True))
        out.append(tile("e4m3", layout, 64, 64, 64, 4, 2, va=1, vb=1, splitk=True))
    for layout in ("TN", "TT"):
        out.append(tile("e4m3", layout, 128, 128, 64, 4, 2))
        out.append(tile("e4m3", layout, 128, 128, 64, 4, 2, va=1, vb=1))
    # LDS-DMA variants: deeper pipelines for the large shapes (2-4 buffers)
    for layout in ("NN", "NT", "TN", "TT"):
        for BM, BN, BK, waves, st in ((256, 256, 64, 4, 2), (256, 256, 64, 8, 2), (256, 256, 32, 4, 3),
                                      (256, 256, 32, 4, 4), (256, 256, 32, 8, 3), (256, 256, 32, 8, 4),
                                      (256, 128, 64, 4, 3), (128, 256, 64, 4, 3), (128, 128, 64, 4, 3),
                                      (128, 128, 64, 4, 4)):
            out.append(dma_tile("bf16", layout, BM, BN, BK, waves, st))
        # split-K for skinny and long-K shapes (a few output blocks, each
        # streaming a slice of K)
        for BM, BN, BK, waves, st in ((64, 256, 64, 4, 2), (64, 128, 64, 4, 3), (128, 128, 64, 4, 3),
                                      (128, 256, 64, 8, 2), (64, 64, 64, 4, 4), (64, 128, 64, 4, 4),
                                      (128, 64, 64, 4, 4), (64, 128, 128, 4, 2)):
            out.append(dma_tile("bf16", layout, BM, BN, BK, waves, st, splitk=True))
        for BM, BN, BK, waves, st in ((256, 256, 64, 4, 2), (128, 128, 64, 4, 3), (256, 256, 32, 4, 4)):
            out.append(dma_tile("f16", layout, BM, BN, BK, waves, st))
        # fp8: BK = 128 (two 64-deep k-steps per k-tile) and 4 waves (with 8,
        # two sets of 32-byte fragments and 128 accumulators per lane exceed
        # the 256 VGPRs of a lane at two waves per SIMD)
        for BM, BN, BK, waves, st in ((256, 256, 128, 4, 2), (256, 128, 128, 4, 3), (128, 128, 128, 4, 3),
                                      (128, 128, 128, 4, 4)):
            out.append(dma_tile("e4m3", layout, BM, BN, BK, waves, st))
    # 16x16x32-block NT tiles (both operands K-major), and the transpose
    # composites built on them
    for dt in ("bf16", "f16"):
        for BM, BN, BK, waves, st in ((256, 256, 64, 8, 2), (256, 128, 64, 4, 3), (128, 256, 64, 4, 3),
                                      (128, 128, 64, 4, 3)):
            if dt == "f16" and BM * BN < 256 * 256:
                continue
            out.append(m16_tile(dt, BM, BN, BK, waves, st))
        out.append(m16_tile(dt, 256, 256, 64, 8, 2, grid=(4, 2)))
        if dt == "bf16":  # 128x128 on 8 waves: two waves per SIMD when a block per CU is all there is
            out.append(m16_tile(dt, 128, 128, 64, 8, 3, grid=(2, 4)))
            out.append(m16_tile(dt, 128, 128, 64, 8, 3, grid=(4, 2)))
            out.append(m16_tile(dt, 128, 128, 64, 8, 5, grid=(4, 2)))
        for layout in ("NN", "TN", "TT"):
            out.append(xpose_tile(dt, layout, 256, 256, 64, 8, 2, m16=True))
            out.append(xpose_tile(dt, layout, 256, 256, 64, 8, 2, m16=True, grid=(4, 2)))
            if dt == "bf16":
                out.append(xpose_tile(dt, layout, 128, 128, 64, 4, 3, m16=True))
                out.append(xpose_tile(dt, layout, 128, 128, 64, 8, 3, m16=True, grid=(2, 4)))
    for BM, BN, BK, waves, st in ((64, 256, 64, 4, 2), (128, 128, 64, 4, 3)):
        out.append(m16_tile("bf16", BM, BN, BK, waves, st, splitk=True))
    # 16x16x32-block NN tiles reading B as stored
    for dt in ("bf16", "f16"):
        for BM, BN, BK, waves, st in ((256, 256, 64, 8, 2), (128, 256, 64, 4, 3), (256, 128, 64, 4, 3),
                                      (128, 128, 64, 4, 3)):
            if dt == "f16" and BM * BN < 256 * 256:
                continue
            out.append(nn16_tile(dt, BM, BN, BK, waves, st))
    for BM, BN, BK, waves, st in ((64, 256, 64, 4, 2), (128, 128, 64, 4, 3)):
        out.append(nn16_tile("bf16", BM, BN, BK, waves, st, splitk=True))
    # 64-column wave tiles: half the register transposes per matrix-core
    # instruction, and 8 waves on a 128x128 block
    for dt in ("bf16", "f16"):
        out.append(nn16_tile(dt, 256, 256, 64, 8, 2, wtn=64))
    out.append(nn16_tile("bf16", 256, 256, 32, 8, 3, wtn=64))
    out.append(nn16_tile("bf16", 256, 256, 32, 8, 4, wtn=64))
    out.append(nn16_tile("bf16", 128, 128, 64, 8, 3, wtn=64))
    # deeper rings for a block per CU: with 4 or 5 32 KB k-tiles in LDS, 3 or
    # 4 are in flight while one is read (the feed from L2 and the last-level
    # cache is bound by bytes in flight at one block per CU)
    out.append(nn16_tile("bf16", 128, 128, 64, 8, 4, wtn=64))
    out.append(nn16_tile("bf16", 128, 128, 64, 8, 5, wtn=64))
    # 32-deep k-tiles, 4 in LDS: the 128x128 winner at two blocks per CU
    # (M = 2048, N = K = 4096); at one block per CU the 64-deep tile wins
    out.append(nn16_tile("bf16", 128, 128, 32, 8, 4, wtn=64))
    out.append(nn16_tile("bf16", 128, 256, 64, 8, 3, wtn=64))
    out.append(nn16_tile("bf16", 128, 128, 64, 8, 3, splitk=True, wtn=64))
    out.append(nn16_tile("bf16", 64, 256, 64, 4, 2, splitk=True, wtn=64))
    # half-height split-K tile for shares that give too few 256x256 tiles
    out.append(nn16_tile("bf16", 128, 256, 64, 8, 3, splitk=True, wtn=64))
    # 128x64 split-K blocks (one column of 4 waves): at M = 128 four k-slices
    # already give 256 blocks, with half the fp32 partial sums of 128x128
    # blocks at eight slices
    out.append(nn16_tile("bf16", 128, 64, 64, 4, 3, splitk=True, wtn=64))
    out.append(nn16_tile("bf16", 128, 64, 64, 4, 4, splitk=True, wtn=64))
    out.append(nn16_tile("bf16", 128, 128, 64, 8, 5, splitk=True, wtn=64))
    # fp8 NT blocks of 256x256 on 8 waves (half-split k-steps, tile_dmah.h),
    # and the transpose composites built on them
    for grid in ((2, 4), (4, 2)):
        out.append(tile("e4m3", "NT", 256, 256, 128, 8, 2, dma=True, grid=grid, half=True))
        out.append(tile("e4m3", "NN", 256, 256, 128, 8, 2, dma=True, xpose=True, grid=grid, half=True))
    for layout in ("TN", "TT"):
        out.append(tile("e4m3", layout, 256, 256, 128, 8, 2, dma=True, xpose=True, grid=(4, 2), half=True))
    out.append(tile("e4m3", "NT", 128, 128, 128, 8, 3, dma=True, grid=(2, 4), half=True))
    out.append(tile("e4m3", "NN", 128, 128, 128, 8, 3, dma=True, xpose=True, grid=(2, 4), half=True))
    # transpose + NT composites for the layouts with an MN-major operand
    for layout in ("NN", "TN", "TT"):
        for BM, BN, BK, waves, st in ((256, 256, 64, 8, 2), (256, 256, 32, 8, 4), (256, 256, 64, 4, 2),
                                      (128, 128, 64, 4, 3)):
            out.append(xpose_tile("bf16", layout, BM, BN, BK, waves, st))
        for BM, BN, BK, waves, st in ((256, 256, 64, 4, 2), (128, 128, 64, 4, 3)):
            out.append(xpose_tile("f16", layout, BM, BN, BK, waves, st))
        for BM, BN, BK, waves, st in ((256, 256, 128, 4, 2), (128, 128, 128, 4, 3)):
            out.append(xpose_tile("e4m3", layout, BM, BN, BK, waves, st))
    # fp32: two tile shapes per layout, each with full-width and 4-byte loads
    for layout in ("NN", "NT", "TN", "TT"):
        for BM, BN, BK in ((128, 128, 16), (64, 64, 32)):
            out.append(tile("f32", layout, BM, BN, BK, 4, 2))
            out.append(tile("f32", layout, BM, BN, BK, 4, 2, va=1, vb=1))
    # small outputs: 32 x 32 blocks with 4 or 8 k-groups of one wave sharing
    # one 256-deep k-tile, so a block keeps a CU's four SIMDs busy
    for dt in ("f32", "bf16"):
        for layout in ("NN", "NT"):
            for wk in (4, 8):
                out.append(tile(dt, layout, 32, 32, 256, 1, 1, wk=wk))
    # fp32 for short K (one or two k-tiles cover it) and 8 waves per block
    for layout in ("NN", "NT"):
        for BM, BN, BK, waves, st in ((64, 64, 64, 4, 1), (128, 128, 32, 8, 2), (128, 64, 32, 8, 2),
                                      (128, 128, 16, 8, 2)):
            out.append(tile("f32", layout, BM, BN, BK, waves, st))
            out.append(tile("f32", layout, BM, BN, BK, waves, st, va=1, vb=1))
    names = [name_of(t) for t in out]
    assert len(set(names)) == len(names), "duplicate candidate names"
    for t in out:
        assert lds_bytes(t) <= 160 * 1024, name_of(t)
    return out


GEMV_KC = {1: 4096, 2: 4096, 4: 2048, 16: 512}  # K rows of A staged in LDS at a time


def gemv(dtype, rows, cw, nw, unroll, mode, splits=(1,), v=None):
    return dict(dtype=dtype, rows=rows, cw=cw, nw=nw, unroll=unroll, mode=mode, splits=tuple(splits),
                v=CH[dtype] if v is None else v)


def gemv_family():
    out = []
    # bf16: M = 1 streams one row of A against all of B; the variants differ in
    # column-block width, waves per workgroup and how K is shared out
    out += [gemv("bf16", 1, 64, 16, 8, 0), gemv("bf16", 1, 128, 16, 8, 0), gemv("bf16", 1, 256, 16, 8, 0),
            gemv("bf16", 1, 64, 8, 16, 0),
            gemv("bf16", 1, 64, 4, 8, 2, (4, 8, 16)), gemv("bf16", 1, 256, 4, 8, 2, (16, 32)),
            gemv("bf16", 1, 64, 4, 8, 1, (4, 8)),
            gemv("bf16", 1, 256, 8, 8, 1, (8, 16, 32)), gemv("bf16", 1, 512, 8, 8, 1, (16, 32, 64)),
            gemv("bf16", 1, 512, 4, 16, 1, (16, 32, 64)), gemv("bf16", 1, 128, 8, 8, 1, (8, 16, 32))]
    # mode 6: up to 16 rows on the 16x16x32 matrix-core instruction (B
    # blocks transposed in registers), K slices summed by a second launch
    out += [gemv_mfma("bf16", 8, 2), gemv_mfma("bf16", 16, 1), gemv_mfma("bf16", 4, 4), gemv_mfma("bf16", 8, 1),
            gemv_mfma("f16", 8, 2), gemv_mfma("f16", 16, 1)]
    # the same kernel registered for 1 and 4 rows (the plan favours the
    # smallest row count that covers M)
    out += [gemv_mfma("bf16", 8, 2, rows=1), gemv_mfma("bf16", 16, 1, rows=1), gemv_mfma("bf16", 8, 2, rows=4),
            gemv_mfma("bf16", 16, 1, rows=4), gemv_mfma("f16", 8, 2, rows=1)]
    # wider workgroups: 2 or 4 blocks of 128 columns, so each reads longer
    # pieces of fewer rows of B
    for rows in (16, 1):
        out += [gemv_mfma("bf16", 16, 1, rows=rows, wn=2), gemv_mfma("bf16", 8, 1, rows=rows, wn=2),
                gemv_mfma("bf16", 16, 1, rows=rows, wn=4), gemv_mfma("bf16", 8, 2, rows=rows, wn=2),
                gemv_mfma("f16", 16, 1, rows=rows, wn=2)]
    # mode 9: the matrix-core GEMV with the slice sum in the same launch
    # (slower than the second launch at N = K = 4096 on the MI355X: each
    # workgroup's device-scope release writes back its XCD's L2)
    for rows in (16, 4, 1):
        out += [gemv_mfma("bf16", 16, 1, rows=rows, fused=True)]
    out += [gemv_mfma("f16", 8, 2, fused=True), gemv_mfma("f16", 8, 2, rows=1, fused=True)]
    # mode 5: mode 4 with the K slices summed by a second launch
    out += [gemv_flat("bf16", 1, 8, 16, sep=True), gemv_flat("bf16", 1, 16, 8, sep=True),
            gemv_flat("bf16", 1, 8, 8, sep=True), gemv_flat("bf16", 1, 4, 16, sep=True),
            gemv_flat("bf16", 4, 8, 8, sep=True), gemv_flat("f16", 1, 8, 16, sep=True),
            gemv_flat("e4m3", 1, 8, 8, sep=True)]
    # mode 4: all of a wave's loads at once
    out += [gemv_flat("bf16", 1, 16, 8), gemv_flat("bf16", 1, 8, 16), gemv_flat("bf16", 1, 16, 16),
            gemv_flat("bf16", 1, 8, 8), gemv_flat("bf16", 1, 4, 16), gemv_flat("bf16", 1, 16, 4),
            gemv_flat("bf16", 4, 8, 8), gemv_flat("f16", 1, 16, 8), gemv_flat("e4m3", 1, 8, 8),
            gemv_flat("e4m3", 1, 4, 16)]
    # mode 3: one workgroup per 32-byte column slice, all of K, siblings that
    # share a 128-byte line on one XCD
    out += [gemv("bf16", 1, 16, 16, 8, 3), gemv("bf16", 1, 16, 8, 16, 3), gemv("bf16", 1, 16, 4, 32, 3),
            gemv("bf16", 4, 16, 8, 8, 3), gemv("f16", 1, 16, 16, 8, 3), gemv("e4m3", 1, 32, 8, 8, 3),
            gemv("e4m3", 4, 32, 4, 8, 3)]
    out += [gemv("bf16", 4, 64, 16, 8, 0), gemv("bf16", 4, 64, 4, 8, 2, (8, 16))]
    out += [gemv("bf16", 16, 64, 4, 4, 0), gemv("bf16", 16, 64, 4, 4, 2, (8, 16)),
            gemv("bf16", 16, 256, 4, 4, 2, (16,)), gemv("bf16", 16, 64, 4, 4, 2, (16,), v=1)]
    out += [gemv("f16", 1, 64, 16, 8, 0), gemv("f16", 1, 64, 4, 8, 2, (8, 16)),
            gemv("f16", 16, 64, 4, 4, 0), gemv("f16", 16, 64, 4, 4, 2, (16,)),
            gemv("f16", 16, 64, 4, 4, 2, (16,), v=1)]
    # (16 waves per workgroup leave 128 VGPRs per lane: too few for 16 rows
    # of accumulators, so the 16-row variants use 8 or 4 waves; fp8 stops at
    # 4 rows, its 16-byte chunks hold 16 columns)
    # fp32: one GEMV, 4-byte loads (any alignment)
    out += [gemv("f32", 16, 64, 8, 4, 0, v=1)]
    out += [gemv("e4m3", 1, 128, 16, 8, 0), gemv("e4m3", 1, 128, 4, 8, 2, (8, 16)),
            gemv("e4m3", 4, 128, 8, 4, 0), gemv("e4m3", 4, 128, 4, 4, 2, (16,)),
            gemv("e4m3", 4, 128, 4, 4, 2, (16,), v=1)]
    # mode 7: rhs stored N x K (NT, TT), up to 16 rows, one launch, no
    # workspace: blocks of 16 B rows on the 16x16 matrix-core instruction
    for dt in ("bf16", "f16"):
        out += [gemv_nt(dt, 1, 8, 8), gemv_nt(dt, 1, 8, 16), gemv_nt(dt, 1, 16, 8), gemv_nt(dt, 2, 8, 8),
                gemv_nt(dt, 1, 4, 16)]
        # the same kernel registered for one row (the plan favours the
        # smallest row count that covers M), so it races the wave-dot form
        out += [gemv_nt(dt, 1, 16, 8, rows=1), gemv_nt(dt, 1, 8, 16, rows=1)]
    out += [gemv_nt("e4m3", 1, 8, 4), gemv_nt("e4m3", 1, 8, 8), gemv_nt("e4m3", 2, 8, 4)]
    # mode 10: the same blocks fed through LDS from coalesced loads (16
    # waves taking 2-unit steps in turn lead at 4 and 16 rows)
    for dt in ("bf16", "f16"):
        out += [gemv_nts(dt, 16, 2), gemv_nts(dt, 16, 4), gemv_nts(dt, 8, 4), gemv_nts(dt, 8, 8)]
        out += [gemv_nts(dt, 16, 2, rows=4)]
    out += [gemv_nts("e4m3", 16, 2), gemv_nts("e4m3", 8, 4), gemv_nts("e4m3", 8, 2)]
    out += [gemv_nts("f32", 16, 2), gemv_nts("f32", 8, 4), gemv_nts("f32", 8, 2)]
    out += [gemv_nt("f32", 1, 8, 8), gemv_nt("f32", 1, 8, 16), gemv_nt("f32", 2, 8, 8)]
    # mode 8: rhs stored N x K, a wave dots whole K-rows of B (1 KiB per load
    # instruction) and reduces across its lanes; 1, 2 or 4 rows of A
    for dt in ("bf16", "f16"):
        out += [gemv_ntdot(dt, 1, 2, 4, 4), gemv_ntdot(dt, 1, 1, 8, 8), gemv_ntdot(dt, 1, 2, 8, 8),
                gemv_ntdot(dt, 1, 4, 4, 2), gemv_ntdot(dt, 2, 2, 4, 4), gemv_ntdot(dt, 4, 2, 4, 4)]
    out += [gemv_ntdot("f32", 1, 2, 4, 4), gemv_ntdot("f32", 1, 1, 8, 8), gemv_ntdot("f32", 4, 2, 4, 4)]
    return out


def gemv_ntdot(dtype, rows, rw, nw, u):
    """MODE 8: `rw` rows of B per wave over all of K, nw waves per workgroup,
    u load instructions deep per row, up to `rows` rows of A."""
    return gemv(dtype, rows, rw, nw, u, 8)


def gemv_nts(dtype, nw, u, rows=16):
    """MODE 10: MODE 7's 16-row blocks with B (and aligned A) loaded as
    contiguous runs and staged through LDS, nw waves taking steps of u units
    in turn; up to `rows` rows of A."""
    return gemv(dtype, rows, 16, nw, u, 10)


def gemv_nt(dtype, nb, nw, u, rows=16):
    """MODE 7: nb blocks of 16 rows of B (outputs) per workgroup, nw waves
    sharing K, u units of K per wave and step; up to `rows` rows of A."""
    return gemv(dtype, rows, 16 * nb, nw, u, 7)


def gemv_launcher(g):
    return "launch_gemv_%s_m%d_c%d_w%d_v%d_u%d_mode%d" % (g["dtype"], g["rows"], g["cw"], g["nw"], g["v"],
                                                         g["unroll"], g["mode"])


def gemv_flat(dtype, rows, nw, r, sep=False):
    """MODE 4: a workgroup covers 64 chunks of columns and nw*r rows of K;
    MODE 5: the same with the K slices summed by a separate launch."""
    return gemv(dtype, rows, 64 * CH[dtype], nw, r, 5 if sep else 4)


def gemv_mfma(dtype, nw, r, rows=16, wn=1, fused=False):
    """MODE 6: wn blocks of 128 columns per workgroup, nw waves (nw / wn per
    column block) of r blocks of 32 rows; up to `rows` rows of A (at most
    16).  MODE 9 (fused): the last K slice of a column block sums the
    slices in the same launch."""
    return gemv(dtype, rows, 128 * wn, nw, r, 9 if fused else 6)


def gemv_name(g, s):
    # narrow-load variant of a type that also has 16-byte ones
    v = "_vb%d" % (g["v"] * E[g["dtype"]]) if (g["v"] != CH[g["dtype"]] and g["dtype"] != "f32") else ""
    if g["mode"] == 7:
        return "gemv_%s_nt_m%d_c%d_w%d_u%d" % (g["dtype"], g["rows"], g["cw"], g["nw"], g["unroll"])
    if g["mode"] == 10:
        return "gemv_%s_nt_m%d_c%d_w%d_u%d_lds" % (g["dtype"], g["rows"], g["cw"], g["nw"], g["unroll"])
    if g["mode"] == 8:
        return "gemv_%s_nt_m%d_r%d_w%d_u%d_dot" % (g["dtype"], g["rows"], g["cw"], g["nw"], g["unroll"])
    base = "gemv_%s_nn_m%d_c%d_w%d%s" % (g["dtype"], g["rows"], g["cw"], g["nw"], v)
    if g["mode"] == 3:
        return base + "_u%d_xcd" % g["unroll"]
    if g["mode"] == 4:
        return base + "_r%d" % g["unroll"]
    if g["mode"] == 5:
        return base + "_r%d_sep" % g["unroll"]
    if g["mode"] == 6:
        return base + "_r%d_mfma" % g["unroll"]
    if g["mode"] == 9:
        return base + "_r%d_mfma_fused" % g["unroll"]
    return base if g["mode"] == 0 else base + ("_f%d" if g["mode"] == 1 else "_p%d") % s


def gemv_lds(g):
    if g["mode"] == 8:
        return 0
    if g["mode"] == 10:
        lch = 2 if g["dtype"] == "e4m3" else 1
        return g["nw"] * 2 * 16 * (4 * lch * g["unroll"] + 1) * 16 + g["nw"] * 16 * 16 * 4
    if g["mode"] == 7:
        return g["nw"] * (g["cw"] // 16) * 256 * 4
    if g["mode"] == 6:
        return g["nw"] * 16 * 128 * 4
    if g["mode"] == 9:
        return g["nw"] * 16 * 128 * 4 + 16
    if g["mode"] in (4, 5):
        return g["nw"] * g["rows"] * g["cw"] * 4 + 16
    if g["mode"] == 3:
        return g["nw"] * g["rows"] * g["cw"] * 4
    return GEMV_KC[g["rows"]] * g["rows"] * 4 + g["nw"] * g["rows"] * g["cw"] * 4 + 16


def generate(outdir, per_file=4):
    os.makedirs(outdir, exist_ok=True)
    gv = gemv_family()
    lst = ["// generated by gen_kernels.py -- do not edit"]
    greg = ["// generated by gen_kernels.py -- do not edit"]
    gdecl = ["// generated by gen_kernels.py -- do not edit", "namespace gt {"]
    seen = set()
    for g in gv:
        fn = gemv_launcher(g)
        assert gemv_lds(g) <= 160 * 1024, fn
        if fn not in seen:
            seen.add(fn)
            lst.append("GT_GEMV(%s, %s, %d, %d, %d, %d, %d, %d, %d)" % (
                fn, TRAITS[g["dtype"]], g["rows"], g["cw"], g["nw"], g["v"], g["unroll"], GEMV_KC[g["rows"]],
                g["mode"]))
            gdecl.append("int %s(const LaunchArgs& a);" % fn)
        # rows a workgroup covers per load step (MODE 4: per K slice)
        if g["mode"] in (7, 8, 10):
            rps = 0  # no K slices
        elif g["mode"] in (6, 9):
            rps = g["nw"] // (g["cw"] // 128) * g["unroll"] * 32
        elif g["mode"] in (4, 5):
            rps = g["nw"] * g["unroll"]
        else:
            rps = (64 // (g["cw"] // CH[g["dtype"]])) * g["nw"]
        for s in g["splits"]:
            greg.append('{"%s", %d, %d, %d, %d, %d, %d, %d, %d, %d, &%s},' % (
                gemv_name(g, s), DT_CODE[g["dtype"]], g["rows"], g["cw"], g["nw"], g["v"] * E[g["dtype"]],
                g["mode"], s, rps, gemv_lds(g), fn))
    gdecl.append("}  // namespace gt")
    _write_if_changed(os.path.join(outdir, "gemv_list.inc"), "\n".join(lst) + "\n")
    _write_if_changed(os.path.join(outdir, "gemv_registry.inc"), "\n".join(greg) + "\n")
    _write_if_changed(os.path.join(outdir, "gemv_decls.inc"), "\n".join(gdecl) + "\n")
    fam = family()
    files = []
    for start in range(0, len(fam), per_file):
        chunk = fam[start:start + per_file]
        lines = ['// generated by gen_kernels.py -- do not edit', '#include "tile_launch.h"', "", "namespace gt {"]
        for t in chunk:
            lines.append("int launch_%s(const LaunchArgs& a) {" % name_of(t))
            m16 = "true" if t["m16"] else "false"
            if t["half"]:
                m16 += ", true"
            if t["xpose"]:
                lines.append("  return tile_xpose_launch<gtk::%s, %d, %d, %d, %d, %d, %d, %s, %s, %s>(a);" % (
                    TRAITS[t["dtype"]], t["BM"], t["BN"], t["BK"], t["WM"], t["WN"], t["ST"],
                    "true" if t["layout"][0] == "T" else "false", "true" if t["layout"][1] == "T" else "false", m16))
                lines.append("}")
                continue
            if t["dma"]:
                lines.append("  return tile_dma_launch<gtk::%s, %d, %d, %d, %d, %d, %d, %s, %s, %s, %s>(a);" % (
                    TRAITS[t["dtype"]], t["BM"], t["BN"], t["BK"], t["WM"], t["WN"], t["ST"],
                    "true" if t["layout"][0] == "T" else "false", "true" if t["layout"][1] == "T" else "false",
                    "true" if t["splitk"] else "false", m16))
                lines.append("}")
                continue
            lines.append("  return tile_launch<gtk::%s, %d, %d, %d, %d, %d, %d, %s, %s, %d, %d, %s, %d>(a);" % (
                TRAITS[t["dtype"]], t["BM"], t["BN"], t["BK"], t["WM"], t["WN"], t["ST"],
                "true" if t["layout"][0] == "T" else "false", "true" if t["layout"][1] == "T" else "false",
                t["VA"], t["VB"], "true" if t["splitk"] else "false", t.get("WK", 1)))
            lines.append("}")
        lines.append("}  // namespace gt")
        path = os.path.join(outdir, "tiles_%03d.hip" % (start // per_file))
        _write_if_changed(path, "\n".join(lines) + "\n")
        files.append(path)
    for old in os.listdir(outdir):  # shards left from a larger family
        path = os.path.join(outdir, old)
        if old.startswith("tiles_") and old.endswith(".hip") and path not in files:
            os.remove(path)
    reg = ["// generated by gen_kernels.py -- do not edit"]
    decl = ["// generated by gen_kernels.py -- do not edit", "namespace gt {"]
    for t in fam:
        n = name_of(t)
        decl.append("int launch_%s(const LaunchArgs& a);" % n)
        reg.append('{"%s", %d, %d, %d, %d, %d, %d, %d, %d, %d, %d, %d, %d, %d, %d, %d, &launch_%s},' % (
            n, DT_CODE[t["dtype"]], LAYOUT_CODE[t["layout"]], t["BM"], t["BN"], t["BK"], t["WM"], t["WN"], t["ST"],
            t["VA"] * E[t["dtype"]], t["VB"] * E[t["dtype"]], 1 if t["splitk"] else 0, lds_bytes(t),
            xpose_bits(t), kernel_family(t), t.get("WK", 1), n))
    decl.append("}  // namespace gt")
    _write_if_changed(os.path.join(outdir, "tile_decls.inc"), "\n".join(decl) + "\n")
    _write_if_changed(os.path.join(outdir, "tile_registry.inc"), "\n".join(reg) + "\n")
    return files


def _write_if_changed(path, text):
    if os.path.exists(path) and open(path).read() == text:
        return
    with open(path, "w") as f:
        f.write(text)


if __name__ == "__main__":
    fam = family()
    print(len(fam), "tile instantiations")
    if len(sys.argv) > 1:
        print("\n".join(generate(sys.argv[1])))
