"""Pins of the oracle's bucket anchor.

The Burn "autotune" page (section on the tuning key, shape bucketing) rounds
each of m, n, k up to a power of the level's base, base^ceil(log_base x):
2.5 at the minimal level, 2 at the balanced level, 1.5 at the extensive
level, the value itself at the full level.  A power that is not an integer
is rounded up.  The oracle does this in exact integer arithmetic; the checks
below take the powers from 80-digit decimal arithmetic instead (a different
route to the same numbers) and hold the oracle to:

* anchor(x) = ceil(v) where v is the smallest power of the base not below x
  (checked at every power's floor, ceiling and their neighbours, and at
  seeded random x up to 2^32 - 1);
* anchor(x) is never below x, and is monotone in x;
* the first integer above each power goes to the next power's ceiling
  (when that power reaches it);
* anything above the last power in range is clamped to 2^32 - 1;
* hand-worked values past the small ones of the wildcard tests: minimal
  2.5^22 = 568,434,188.608...: 568,434,188 -> 568,434,189 and 568,434,189 ->
  ceil(2.5^23 = 1,421,085,471.52...) = 1,421,085,472; extensive 1.5^40 =
  11,057,332.32...: 11,057,332 -> 11,057,333 and 11,057,333 ->
  ceil(1.5^41 = 16,585,998.48...) = 16,585,999.
"""
import bisect
import random
from decimal import ROUND_CEILING, Decimal, getcontext

import pytest

from oracle import key as ok

TOP = 0xFFFFFFFF
BASES = {"minimal": "2.5", "balanced": "2", "extensive": "1.5"}


def powers(level):
    """base^j (80-digit decimals), j = 0, 1, ..., up to the first beyond 2^32 - 1."""
    getcontext().prec = 80
    b, v, out = Decimal(BASES[level]), Decimal(1), []
    while True:
        out.append(v)
        if v > TOP:
            return out
        v *= b


def ceil_dec(v):
    return int(v.to_integral_value(rounding=ROUND_CEILING))


def expected(pw, x):
    j = bisect.bisect_left(pw, Decimal(x))  # smallest power >= x
    return min(ceil_dec(pw[j]), TOP)


@pytest.mark.parametrize("level", sorted(BASES))
def test_anchor_is_the_rounded_smallest_power_not_below(level):
    pw = powers(level)
    xs = set()
    for v in pw:
        c = ceil_dec(v)
        xs.update(x for x in (c - 2, c - 1, c, c + 1) if 1 <= x <= TOP)
    rng = random.Random(5)
    xs.update(rng.randint(1, TOP) for _ in range(20000))
    xs.update((TOP, TOP - 1))
    xs = sorted(xs)
    got = [ok.anchor(x, level) for x in xs]
    for x, g in zip(xs, got):
        assert g == expected(pw, x), (level, x)
        assert g >= x
    assert all(got[i] <= got[i + 1] for i in range(len(got) - 1))


@pytest.mark.parametrize("level", sorted(BASES))
def test_values_in_range_and_clamp(level):
    pw = [v for v in powers(level) if v <= TOP]
    # the first integer above a power goes to the next power's ceiling when
    # that power reaches it (with base 1.5 no integer lies in (1, 1.5], so
    # ceil(1.5) = 2 is never a bucket: 2 -> ceil(2.25) = 3)
    assert ok.anchor(1, level) == 1
    for prev, v in zip(pw, pw[1:]):
        x = int(prev) + 1
        want = ceil_dec(v) if x <= v else None
        if want is not None:
            assert ok.anchor(x, level) == want
            assert ok.anchor(int(v), level) == want
    assert ok.anchor(ceil_dec(pw[-1]) + 1, level) == TOP
    assert ok.anchor(TOP, level) == TOP


def test_hand_worked_large_buckets():
    assert ok.anchor(568434188, "minimal") == 568434189
    assert ok.anchor(568434189, "minimal") == 1421085472
    assert ok.anchor(11057332, "extensive") == 11057333
    assert ok.anchor(11057333, "extensive") == 16585999
    assert ok.anchor(2 ** 31, "balanced") == 2 ** 31 and ok.anchor(2 ** 31 + 1, "balanced") == TOP
    assert ok.anchor(7, "full") == 7 and ok.anchor(2 ** 40, "full") == TOP
    with pytest.raises(ValueError):
        ok.anchor(0)
