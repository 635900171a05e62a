"""Reference reader of the tuning-results file.  TEST INFRASTRUCTURE ONLY.

Format after the PyTorch TunableOp guide, section 3.2 (CSV results file:
"Validator" lines, then one row per tuned op with op name, parameters,
solution and an optional average time; a validator mismatch rejects the
whole file; setting the solution to the default implementation by hand forces
the fallback), combined with the per-entry checksum of the Burn "autotune"
page, section "第一次遇到一个键" (first time a key is seen: an entry carries the
hash of all candidate names it was tuned against, and is ignored when the
candidate list has changed).

  Validator,<NAME>,<value>          one per validator
  GemmTuned,<compact key text>,<candidate name>,<median us or empty>,<checksum>

* Every validator the reader expects must be present with the expected value,
  else the whole file is rejected.
* A row whose checksum differs from the current checksum of its input-type
  candidate set, whose candidate name is not in that set, or that does not
  parse, is skipped (and counted).
* Blank lines and lines starting with '#' are ignored; a later row for the
  same key replaces an earlier one.
* Checksum (a reading: the page names only "a hash of all the names
  concatenated"): 64-bit FNV-1a over the candidate names joined by '\\n', in
  registration order, printed as 16 lowercase hex digits.
"""
from . import key as okey

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3


def fnv1a64(data: bytes) -> int:
    h = FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def checksum(names):
    return "%016x" % fnv1a64("\n".join(names).encode())


class Rejected(Exception):
    pass


def read(text, expected_validators, candidate_sets):
    """Parse a results file.

    expected_validators: {name: value} the reader requires.
    candidate_sets: {input dtype: [candidate names in registration order]}.
    Returns (table, skipped) with table {compact key text: (name, median_us)}.
    Raises Rejected when a validator is missing or differs."""
    seen = {}
    rows = []
    for line in text.splitlines():
        s = line.strip()
        if not s or s.startswith("#"):
            continue
        fields = s.split(",")
        if fields[0] == "Validator":
            if len(fields) != 3:
                raise Rejected("malformed validator line")
            seen[fields[1]] = fields[2]
        elif fields[0] == "GemmTuned":
            rows.append(fields)
    for name, value in expected_validators.items():
        if seen.get(name) != value:
            raise Rejected("validator %s: file %r, expected %r" % (name, seen.get(name), value))
    sums = {d: checksum(n) for d, n in candidate_sets.items()}
    table, skipped = {}, 0
    for f in rows:
        if len(f) != 5:
            skipped += 1
            continue
        try:
            fields = okey.parse_compact(f[1])
        except ValueError:
            skipped += 1
            continue
        d = fields["elem_lhs"]
        if d not in candidate_sets or f[4] != sums[d] or f[2] not in candidate_sets[d]:
            skipped += 1
            continue
        med = None
        if f[3] != "":
            try:
                med = float(f[3])
            except ValueError:
                skipped += 1
                continue
        table[okey.compact_text(fields)] = (f[2], med)
    return table, skipped


# ---------------------------------------------------------------- untuned file
# The record of problems that missed while tuning was off (TunableOp guide,
# section 6.2, step 1: the untuned GEMMs are collected into a file that a
# second step tunes).  The guide names the file and what a row carries (the
# op, its type and transposes, M/N/K and the leading dimensions) but not its
# exact columns; the reading here is one row per problem:
#   GemmUntuned,<compact key>,<in type>,<out type>,<layout>,M,N,K,lda,ldb,ldc,<A addr % 256>,<B addr % 256>
# Blank lines, '#' lines and rows of other kinds are ignored.

UNTUNED_COLUMNS = ("key", "in_dtype", "out_dtype", "layout", "M", "N", "K", "lda", "ldb", "ldc", "off_a", "off_b")


def read_untuned(text):
    """The GemmUntuned rows of an untuned file as dicts keyed by
    UNTUNED_COLUMNS (numbers as int).  Raises ValueError on a row with the
    wrong column count, an unknown type or layout, a non-positive size or an
    offset outside 0..255."""
    rows = []
    for line in text.splitlines():
        s = line.strip()
        if not s or s.startswith("#"):
            continue
        f = s.split(",")
        if f[0] != "GemmUntuned":
            continue
        if len(f) != 1 + len(UNTUNED_COLUMNS):
            raise ValueError("untuned row with %d columns" % len(f))
        r = dict(zip(UNTUNED_COLUMNS, f[1:]))
        if r["in_dtype"] not in okey.DTYPES or r["out_dtype"] not in okey.DTYPES:
            raise ValueError("bad type in %r" % s)
        if r["layout"] not in ("NN", "NT", "TN", "TT"):
            raise ValueError("bad layout in %r" % s)
        for c in UNTUNED_COLUMNS[4:]:
            r[c] = int(r[c])
        if min(r[c] for c in UNTUNED_COLUMNS[4:10]) < 1 or not (0 <= r["off_a"] < 256 and 0 <= r["off_b"] < 256):
            raise ValueError("bad size or offset in %r" % s)
        okey.parse_compact(r["key"])
        rows.append(r)
    return rows
