"""The oracle's streaming steps pinned to independent facts: the gradient
sum against Python's exactly rounded math.fsum and integer closed forms,
the weight copy against bit identity, the gather against a hand-worked
permutation and numpy's take."""
import math

import numpy as np

import oracle


def test_grad_reduce_matches_fsum():
    rng = np.random.default_rng(0)
    for n_rep in range(0, 5):
        master = (rng.standard_normal(500) * 0.02).astype(np.float32)
        reps = [(rng.standard_normal(500) * 0.02).astype(np.float32)
                for _ in range(n_rep)]
        got = oracle.grad_reduce(master, reps)
        for i in range(500):
            terms = [float(master[i])] + [float(r[i]) for r in reps]
            want = math.fsum(terms)
            bound = 8 * 2.0 ** -53 * sum(abs(t) for t in terms)
            assert abs(got[i] - want) <= bound


def test_grad_reduce_closed_forms():
    # integers are summed exactly: 3 + 1 + 2 + 4 = 10
    m = np.full(7, 3.0, np.float32)
    reps = [np.full(7, v, np.float32) for v in (1.0, 2.0, 4.0)]
    assert np.all(oracle.grad_reduce(m, reps) == 10.0)
    # no replica: the master is unchanged
    assert np.array_equal(oracle.grad_reduce(m, []), m.astype(np.float64))
    # cancellation is exact in float64: 1 + 2^-24 - 1 = 2^-24
    r = oracle.grad_reduce(np.ones(1, np.float32),
                           [np.full(1, 2.0 ** -24, np.float32),
                            -np.ones(1, np.float32)])
    assert r[0] == 2.0 ** -24
    # replicas enter with their sign and each exactly once
    r = oracle.grad_reduce(np.zeros(1, np.float32),
                           [np.full(1, 5.0, np.float32),
                            np.full(1, -2.0, np.float32)])
    assert r[0] == 3.0


def test_weight_sync_is_a_bitwise_copy():
    w = np.array([0x3F80, 0xFFFF, 0x0001, 0x7F80], np.uint16)
    reps = oracle.weight_sync(w, 3)
    assert len(reps) == 3
    for r in reps:
        assert r.dtype == np.uint16 and np.array_equal(r, w)
    reps[0][0] = 0
    assert w[0] == 0x3F80 and reps[1][0] == 0x3F80, "independent copies"
    assert oracle.weight_sync(w, 0) == []


def test_gather_hand_worked():
    # 3 tokens, k = 2: assignments 0..5 come from tokens 0,0,1,1,2,2
    x = np.array([[10, 11], [20, 21], [30, 31]], np.int16)
    perm = np.array([5, 0, 3, 1, 4, 2])
    out = oracle.gather(x, perm, 2)
    assert out.tolist() == [[30, 31], [10, 11], [20, 21], [10, 11],
                            [30, 31], [20, 21]]
    rng = np.random.default_rng(1)
    x = rng.integers(-1000, 1000, size=(50, 8)).astype(np.int16)
    perm = rng.permutation(150)
    assert np.array_equal(oracle.gather(x, perm, 3),
                          np.take(x, perm // 3, axis=0))


def test_grad_reduce_rounded_order_and_rounding():
    """The binary32 result of the binary64 left-to-right sum.
    (1 + 2^-24) + 2^-24 is carried exactly and rounds to 1 + 2^-23, where a
    binary32 running sum would tie to even twice and give 1; 1 + 2^-60 - 1
    gives 0 left to right (1 + 2^-60 rounds to 1 in binary64), where the
    exact sum or another order gives 2^-60. On terms whose binary64 partial
    sums are exact (magnitudes within 2^-10 .. 2^-3), every result is the
    correctly rounded binary32 of the exact sum, checked with fractions."""
    from fractions import Fraction
    u = np.float32(2.0 ** -24)
    got = oracle.grad_reduce_rounded(np.ones(3, np.float32),
                                     [np.full(3, u), np.full(3, u)])
    assert got.dtype == np.float32
    assert np.all(got == np.float32(1.0 + 2.0 ** -23))
    got = oracle.grad_reduce_rounded(np.ones(1, np.float32),
                                     [np.full(1, 2.0 ** -60, np.float32),
                                      -np.ones(1, np.float32)])
    assert got[0] == 0.0
    got = oracle.grad_reduce_rounded(np.ones(1, np.float32),
                                     [-np.ones(1, np.float32),
                                      np.full(1, 2.0 ** -60, np.float32)])
    assert got[0] == np.float32(2.0 ** -60)

    def round_f32(q):
        # nearest float32 to the rational q, ties to even (normal range)
        f = np.float32(float(q))
        if Fraction(float(f)) == q:
            return f
        g = np.nextafter(f, np.float32(np.inf) if Fraction(float(f)) < q
                         else np.float32(-np.inf))
        lo, hi = sorted((f, g))
        dl, dh = abs(Fraction(float(lo)) - q), abs(Fraction(float(hi)) - q)
        if dl != dh:
            return lo if dl < dh else hi
        return lo if int(np.array(lo).view(np.int32)) % 2 == 0 else hi

    rng = np.random.default_rng(2)

    def terms(n):
        mag = 2.0 ** rng.uniform(-10, -3, n)
        return (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)

    master = terms(400)
    reps = [terms(400) for _ in range(4)]
    got = oracle.grad_reduce_rounded(master, reps)
    for i in range(400):
        q = Fraction(float(master[i])) + sum(Fraction(float(r[i]))
                                             for r in reps)
        assert got[i] == round_f32(q), i
    # with no replica the master comes back unchanged
    assert np.array_equal(oracle.grad_reduce_rounded(master, []), master)
