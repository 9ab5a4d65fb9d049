"""The lambda attention kernel leaves out the exponentials of a skipped tile when
they cannot change its row sum.  These checks pin the fp32 facts that rule rests
on, in numpy float32 and in the kernel's summation order (host arithmetic only):

1. 2^a rounds to +0 in fp32 for every a below -150 (the smallest subnormal is
   2^-149), so exp2 of an argument under the kernel's -200 gives +0.
2. A lane adds at most 32 terms per tile, each at most 2^arg, summed pairwise as
   the kernel does.  With l in [2^(E-1), 2^E) (frexp's exponent E) and
   arg < E - 31 the sum stays below a quarter of an ulp of l, and the fp32
   result of l + that sum is l.  The step of margin is needed: at arg = E - 30
   the bound is exactly half an ulp, and an exp2 result a little above the true
   value then changes l.
"""

import numpy as np

F32 = np.float32
EXP2_OVERSHOOT = F32(1.0 + 2.0 ** -21)  # exp2 within two ulps above the true value


def kernel_sum(p):
    """The row-sum of one lane's 32 exponentials, in the kernel's order: pairs of
    s0 and s1 entries, then a balanced tree over the eight partial sums."""
    p = np.asarray(p, dtype=F32)
    s0, s1 = p[:16], p[16:]
    ps = [F32(F32(s0[2 * i] + s0[2 * i + 1]) + F32(s1[2 * i] + s1[2 * i + 1])) for i in range(8)]
    a = F32(F32(ps[0] + ps[1]) + F32(ps[2] + ps[3]))
    b = F32(F32(ps[4] + ps[5]) + F32(ps[6] + ps[7]))
    return F32(a + b)


def exponent(l):
    return int(np.frexp(F32(l))[1])  # l in [2^(E-1), 2^E)


def test_exp2_below_minus_150_rounds_to_zero():
    for a in (-150.5, -151.0, -160.0, -200.0, -1000.0):
        assert F32(2.0 ** a) == 0.0
    assert F32(2.0 ** -149) > 0.0  # the smallest subnormal itself is not zero


def test_terms_below_half_an_ulp_leave_the_sum_unchanged():
    rng = np.random.default_rng(7)
    for _ in range(20000):
        E = int(rng.integers(-30, 60))
        # l anywhere in its binade, the low end (the largest relative effect) included
        l = F32(2.0 ** (E - 1) * (1.0 + (0.0 if rng.random() < 0.2 else rng.random())))
        if not (2.0 ** (E - 1) <= float(l) < 2.0 ** E):
            continue
        assert exponent(l) == E
        arg = (E - 31) - (0.0 if rng.random() < 0.3 else rng.random() * 20.0)
        top = F32(F32(2.0 ** arg) * EXP2_OVERSHOOT)
        # the worst case: every term at its largest, or random terms below it
        p = np.full(32, top, dtype=F32) if rng.random() < 0.5 else (rng.random(32) * top).astype(F32)
        assert F32(l + kernel_sum(p)) == l


def test_the_margin_matters():
    for E in (-10, 0, 1, 7, 30):
        l = F32(2.0 ** (E - 1))  # the low end of the binade: the largest relative effect
        # at the kernel's bound every term may sit an ulp or two above 2^arg
        top = F32(F32(2.0 ** (E - 31)) * EXP2_OVERSHOOT)
        assert F32(l + kernel_sum(np.full(32, top, dtype=F32))) == l
        # one step less margin is exactly half an ulp: an overshooting exp2 changes l
        top = F32(F32(2.0 ** (E - 30)) * EXP2_OVERSHOOT)
        assert F32(l + kernel_sum(np.full(32, top, dtype=F32))) != l
        # and without the factor for 32 terms the sum changes l outright
        top = F32(2.0 ** (E - 26))
        assert F32(l + kernel_sum(np.full(32, top, dtype=F32))) != l
