"""Reference group and priority rules.  TEST INFRASTRUCTURE ONLY.

The Burn "autotune" page describes how a plan is built from priorities (see
select.py) but its table of per-group rules did not survive extraction; only
the inputs it reads are named (the key's size class and shape class).  The
rules below are this library's reading, written out independently of the GPU
library so the library's plan can be checked against it bit for bit.  What
the pages do state about plans pins them (tests/test_oracle_plan_pins.py):
the fallback is the first candidate and the last resort; unsupported
candidates are demoted, not removed, and a wholly demoted group is still
tried whole before the next group (the page's wgpu/WGSL example); decode
with 16 rows gets a 16-row candidate in the first round and a 128-row block
is not among the first round's plain tiles (CMU 15-779 Lecture 9 notes,
section 2.2); a 512 x 512 output with a long K races the 16-slice split-K
in the first round (same section).  The thresholds themselves (64 output
blocks, 4 * slices * BK, twice the problem side) are readings the pages do
not fix.

Groups, in registration order: naive, gemv, tile.
  naive  MIN always (the fallback that always works)
  gemv   MAX when the bucketed m is 1, else NEVER (skipped)
  tile   HIGH
A GEMV candidate also belongs to the tile group, so for 1 < M <= 16 it races
the tiles there.

In-group priority of a candidate for a key:
  * NEVER if its layout does not match (GEMV: built for the rhs stored as
    is or for the rhs stored transposed, either lhs; tiles: built for one
    layout; naive: any).
  * naive: MIN.
  * "narrow" candidates (loads narrower than 16 bytes where 16-byte ones
    exist) drop to MEDIUM when both stride factors allow 16-byte loads.
  * GEMV: NEVER if it handles fewer rows than the bucketed m; HIGH if its
    row count is the smallest row count that covers m among its type's GEMV
    kernels for the key's layout, else MEDIUM.
  * split-K tiles: NEVER unless the output has at most 64 of its blocks and
    the bucketed k is at least 4 * slices * BK; then HIGH.
  * tiles of at most 32 x 32 outputs (the blocks whose k-groups share one
    k-tile): NEVER when the output has more than 256 of them (more blocks
    than CUs: larger blocks reuse their operands better there) or the
    bucketed k is above 4 * BK (a long walk of k-tiles, one at a time).
  * other tiles: MEDIUM when a block side above 64 is at least twice the
    bucketed problem side, else HIGH.
Supported (else demoted to MIN): the stride factors allow the candidate's
load widths (ctz >= log2 bytes), its LDS use fits 160 KB, the output is not
fp8.
"""
from .select import HIGH, MAX, MEDIUM, MIN, NEVER

GROUPS = ("naive", "gemv", "tile")


def log2i(x):
    r = 0
    while (1 << r) < x:
        r += 1
    return r


def group_priority(group, key):
    if group == "naive":
        return MIN
    if group == "gemv":
        return MAX if key["m"] == 1 else NEVER
    return HIGH


def is_narrow(c):
    if c["group"] == 0:
        return False
    if c["group"] == 1:
        return c["vb_bytes"] < 16 and c["dtype"] != "f32"
    return c["va_bytes"] < 16 or c["vb_bytes"] < 16


def layout_code(key):
    return (2 if key["layout_lhs"] != "Contiguous" else 0) | (1 if key["layout_rhs"] != "Contiguous" else 0)


def layout_ok(c, lay):
    """A candidate's layout code: -1 any, -2 rhs stored as is (lhs either),
    -3 rhs stored transposed (lhs either), else exactly that layout."""
    if c["layout"] == -1:
        return True
    if c["layout"] == -2:
        return (lay & 1) == 0
    if c["layout"] == -3:
        return (lay & 1) == 1
    return c["layout"] == lay


def cand_priority(c, key, cands):
    lay = layout_code(key)
    if not layout_ok(c, lay):
        return NEVER
    if c["group"] == 0:
        return MIN
    narrow = MEDIUM if (is_narrow(c) and key["lhs_stride"] >= 4 and key["rhs_stride"] >= 4) else HIGH
    m, n, k = key["m"], key["n"], key["k"]
    if c["group"] == 1:
        if c["rows"] < m:
            return NEVER
        fit = min(o["rows"] for o in cands if o["group"] == 1 and layout_ok(o, lay) and o["rows"] >= m)
        return min(HIGH if c["rows"] == fit else MEDIUM, narrow)
    if c["splitk"] > 1:
        tiles = -(-m // c["BM"]) * -(-n // c["BN"])
        if tiles > 64 or k < 4 * c["splitk"] * c["BK"]:
            return NEVER
        return narrow
    if c["BM"] * c["BN"] <= 32 * 32 and (-(-m // c["BM"]) * -(-n // c["BN"]) > 256 or k > 4 * c["BK"]):
        return NEVER
    p = HIGH
    if (c["BM"] > 64 and c["BM"] >= 2 * m) or (c["BN"] > 64 and c["BN"] >= 2 * n):
        p = MEDIUM
    return min(p, narrow)


def supported(c, key):
    if c["va_bytes"] > 1 and key["lhs_stride"] < log2i(c["va_bytes"]):
        return False
    if c["vb_bytes"] > 1 and key["rhs_stride"] < log2i(c["vb_bytes"]):
        return False
    if c["lds_bytes"] > 160 * 1024:
        return False
    if key["elem_out"] == "e4m3":
        return False
    return True


def plan(key, cands):
    """Rounds of candidate indices for a key; cands: list of dicts with the
    fields of the library's candidate description (name, group 0/1/2, dtype,
    layout, BM, BN, BK, splitk, va_bytes, vb_bytes, rows, lds_bytes)."""
    from .select import build_plan
    gp = {g: group_priority(g, key) for g in GROUPS}
    groups = [["naive"] if c["group"] == 0 else (["gemv", "tile"] if c["group"] == 1 else ["tile"]) for c in cands]
    prio = [cand_priority(c, key, cands) for c in cands]
    sup = [supported(c, key) for c in cands]
    return build_plan(gp, groups, prio, sup)
