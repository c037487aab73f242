"""The column-major 2-D orders at d_state 16 find the patch row of visit step q
as (q mod H) W + q div H, with the quotient taken from the fp32 product
q * (1/H) truncated to an integer and corrected by at most one each way.  The
host sends a grid down that path only below 2^23 steps.  This emulates that
arithmetic exactly in IEEE fp32 (round to nearest for the reciprocal and the
product, truncation for the conversion, as the GPU does them) and checks it
against integer divmod, over whole grids and random steps of random grids up
to the limit: the claim the size limit rests on."""
import numpy as np

LIMIT = 1 << 23


def fp32_divmod(q, H):
    inv = np.float32(1.0) / np.float32(H)
    qd = (q.astype(np.float32) * inv).astype(np.int64)    # q >= 0: truncation is floor
    qm = q - qd * H
    lo = qm < 0
    qm[lo] += H
    qd[lo] -= 1
    hi = qm >= H
    qm[hi] -= H
    qd[hi] += 1
    return qd, qm


def test_whole_grids_are_permutations():
    for H, W in [(2, 3), (4, 4), (7, 7), (19, 23), (45, 47), (56, 56), (64, 128), (3, 2796202),
                 (2796202, 3), (8191, 1024)]:
        L = H * W
        assert L < LIMIT
        q = np.arange(L, dtype=np.int64)
        qd, qm = fp32_divmod(q, H)
        assert np.array_equal(qd, q // H) and np.array_equal(qm, q % H), (H, W)
        rows = qm * W + qd
        assert np.array_equal(np.sort(rows), q)


def test_random_grids_up_to_the_limit():
    rng = np.random.default_rng(23)
    for _ in range(400):
        H = int(rng.integers(2, LIMIT // 2))
        W = int(rng.integers(2, max(3, (LIMIT - 1) // H + 1)))
        if H * W >= LIMIT:
            continue
        q = np.concatenate([rng.integers(0, H * W, size=2048, dtype=np.int64),
                            np.array([0, H - 1, H, H * W - 1], dtype=np.int64)])
        qd, qm = fp32_divmod(q, H)
        assert np.array_equal(qd, q // H) and np.array_equal(qm, q % H), H


def test_steps_just_below_the_limit():
    # the largest steps allowed, for divisors near powers of two and primes
    q = np.arange(LIMIT - 4096, LIMIT, dtype=np.int64)
    for H in (2, 3, 5, 7, 127, 128, 129, 4095, 4097, 65521, 1 << 20, (1 << 22) - 3):
        qd, qm = fp32_divmod(q, H)
        assert np.array_equal(qd, q // H) and np.array_equal(qm, q % H), H
