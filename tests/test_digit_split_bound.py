"""The int8 digit split behind the digit-score attention, checked on the CPU in exact arithmetic
(no GPU code is run or imported): the split of an f32 row into seven base-128 digits with one
power-of-two exponent, and the error of a dot product formed from the digit pairs t + u <= 6.
This pins the bound the reading rests on: the kept pairs and the split's remainders leave at
most 2^-41 * 2^(Eq+Ek) of q . k (Ozaki, Ogita, Oishi, Rump, Numerical Algorithms 59, 2012, for
the error-free splitting; the digit rule is the one the q/k epilogue and the append apply)."""
from fractions import Fraction

import numpy as np

T = 7


def split(row):
    """Exponent E and digits D[t][d] of an f32 row, every step an exact f32 operation: x = row *
    2^-E (|x| < 1/2), then seven times y = 128 x, D = round-half-even(y), x = y - D."""
    row = np.asarray(row, np.float32)
    amax = float(np.max(np.abs(row)))
    if amax == 0.0:
        return 0, np.zeros((T, row.size), np.int64)
    E = int(np.frexp(np.float32(amax))[1]) + 1
    x = np.ldexp(row, -E).astype(np.float32)
    digits = []
    for _ in range(T):
        y = (x * np.float32(128)).astype(np.float32)
        r = np.rint(y)
        digits.append(r.astype(np.int64))
        x = (y - r).astype(np.float32)
    return E, np.array(digits)


def exact(v):
    return [Fraction(float(a)) for a in np.asarray(v, np.float32)]


def split_dot(Eq, Dq, Ek, Dk):
    """sum over t + u <= 6 of 128^-(t+u+2) Dq_t . Dk_u, times 2^(Eq+Ek), exactly."""
    acc = 0
    for t in range(T):
        for u in range(T - t):
            acc += int(np.dot(Dq[t], Dk[u])) * 128 ** (6 - t - u)
    return Fraction(acc) * Fraction(2) ** (Eq + Ek) / Fraction(128) ** 8


def bound(Eq, Ek, n):
    """Dropped diagonals d = 7..12 (13 - d pairs, |D| <= 64) and the remainders (|rho| <= 2^-50
    per element against a digit sum of magnitude <= 1/2), for n dims, times 2^(Eq+Ek)."""
    drop = sum((13 - d) * 64 * 64 * n * Fraction(1, 128 ** (d + 2)) for d in range(7, 13))
    rem = n * (2 * Fraction(1, 2) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 100))
    return (drop + rem) * Fraction(2) ** (Eq + Ek)


def rows(rng, n, count):
    """Rows like normalized, rotated queries and keys, and harder ones: a wide spread of
    magnitudes within a row, exact powers of two at the maximum, zeros, a single nonzero."""
    out = []
    for i in range(count):
        kind = i % 5
        if kind == 0:
            r = rng.standard_normal(n)
        elif kind == 1:
            r = rng.standard_normal(n) * 10.0 ** rng.uniform(-12, 2, n)
        elif kind == 2:
            r = rng.standard_normal(n)
            r[rng.integers(n)] = 2.0 ** int(rng.integers(-20, 20))
        elif kind == 3:
            r = np.where(rng.random(n) < 0.5, 0.0, rng.standard_normal(n)) * 2.0 ** int(rng.integers(-30, 30))
        else:
            r = np.zeros(n)
            r[rng.integers(n)] = rng.standard_normal()
        out.append(r.astype(np.float32))
    return out


def test_digits_in_range_and_row_reconstructed():
    rng = np.random.default_rng(11)
    for r in rows(rng, 128, 200):
        E, D = split(r)
        assert np.all(np.abs(D) <= 64)
        if not np.any(r):
            assert E == 0 and not np.any(D)
            continue
        for d, v in enumerate(exact(r)):
            approx = sum(Fraction(int(D[t][d]), 128 ** (t + 1)) for t in range(T)) * Fraction(2) ** E
            assert abs(v - approx) <= Fraction(2) ** (E - 50)


def test_split_dot_within_the_bound_and_sums_fit_int32():
    rng = np.random.default_rng(12)
    qs, ks = rows(rng, 128, 120), rows(rng, 128, 120)
    worst = Fraction(0)
    for q, k in zip(qs, ks):
        Eq, Dq = split(q)
        Ek, Dk = split(k)
        for d in range(2 * T - 1):  # every diagonal's integer sum fits int32 with room
            s = sum(int(np.dot(Dq[t], Dk[d - t])) for t in range(max(0, d - T + 1), min(T, d + 1)))
            assert abs(s) < 2 ** 31
        ref = sum(a * b for a, b in zip(exact(q), exact(k)))
        err = abs(split_dot(Eq, Dq, Ek, Dk) - ref)
        b = bound(Eq, Ek, 128)
        assert err <= b
        if b:
            worst = max(worst, err / b)
    assert worst < 1  # and the stated 2^-41 * 2^(Eq+Ek) is that bound to within 1%
    assert abs(bound(0, 0, 128) * 2 ** 41 - 1) < 0.01


def test_planted_mistakes_are_caught():
    """The check has teeth: each plausible slip in the combine leaves an error above the bound
    (pairs of diagonal 5 left out, an exponent off by one, one pair's sign flipped)."""
    rng = np.random.default_rng(13)
    unit = Fraction(1) / Fraction(128) ** 8
    for _ in range(20):
        q, k = rng.standard_normal(128).astype(np.float32), rng.standard_normal(128).astype(np.float32)
        Eq, Dq = split(q)
        Ek, Dk = split(k)
        scale = Fraction(2) ** (Eq + Ek)
        good = split_dot(Eq, Dq, Ek, Dk)
        diag5 = sum(int(np.dot(Dq[t], Dk[5 - t])) for t in range(6)) * 128 * unit * scale
        pair01 = int(np.dot(Dq[0], Dk[1])) * 128 ** 5 * unit * scale
        ref = sum(a * b for a, b in zip(exact(q), exact(k)))
        b = bound(Eq, Ek, 128)
        assert abs(good - ref) <= b
        assert abs(good - diag5 - ref) > b
        assert abs(good / 2 - ref) > b
        assert abs(good - 2 * pair01 - ref) > b
