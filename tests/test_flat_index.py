"""Host-side checks of the index arithmetic in the flat backward kernel over a
non-last axis (lse_grad_flat in lse_dim.hip), on the CPU.

The kernel divides 32-bit numerators exactly by a runtime divisor d with a
precomputed 64-bit multiplier m = floor((2^64 - 1) / d) + 1: floor(a / d) is
the high 64 bits of m * a for every a, d < 2^32 (Lemire, Kaser and Kurz,
"Faster Remainder by Direct Computation", 2019, the 64-bit multiplier for
32-bit operands). d = 1 would need m = 2^64, so the host passes m = 0 for it
and the kernel then returns a itself.

Each workgroup locates its first flat element F with 64-bit divisions, and
the element d places later (d below the chunk of CH elements) by its column
and the rows and slices it lies past F's: where inner > CH a single compare
(one wrap at most, to the next row or, from a slice's last row, the next
slice); else slot m * 256 + t steps column and row by 256 elements from one
exact division, and the slice is a division unless the array has one slice.
Written out here as in the kernel and compared with the direct index
(f div (n * inner)) * inner + f mod inner of every element of random chunks.
"""
import numpy as np
import pytest

U64 = (1 << 64) - 1


def magic(d: int) -> int:
    return 0 if d == 1 else U64 // d + 1


def fastdiv(a: int, m: int) -> int:
    return a if m == 0 else (m * a) >> 64


@pytest.mark.parametrize("d", [1, 2, 3, 5, 7, 10, 641, 4097, 50257, 65535, 65536, 1000003,
                               (1 << 31) - 1, 1 << 31, (1 << 32) - 3, (1 << 32) - 1])
def test_fastdiv_is_exact(d):
    m = magic(d)
    rng = np.random.default_rng(d)
    cases = [0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, (1 << 32) - 1, (1 << 32) - 2,
             ((1 << 32) - 1) // d * d, ((1 << 32) - 1) // d * d - 1]
    cases += [int(v) for v in rng.integers(0, 1 << 32, size=4000, dtype=np.uint64)]
    for a in cases:
        if 0 <= a < (1 << 32):
            assert fastdiv(a, m) == a // d, (a, d)


def test_fastdiv_random_divisors():
    rng = np.random.default_rng(7)
    for d in rng.integers(2, 1 << 32, size=300, dtype=np.uint64):
        d = int(d)
        m = magic(d)
        for a in rng.integers(0, 1 << 32, size=50, dtype=np.uint64):
            a = int(a)
            assert fastdiv(a, m) == a // d, (a, d)


def locate_chunk(F: int, CH: int, n: int, inner: int, total: int) -> list:
    """The kernel's lookup index for the slots d = m * 256 + t of the chunk at
    F (elements F + d < total), in its two cases."""
    qF = F // inner
    iF = F - qF * inner
    oF = qF // n
    jF = qF - oF * n
    M = CH // 256
    out = {}
    if inner > CH:
        gF = oF * inner + iF
        last_row = jF + 1 == n
        for d in range(CH):
            if d < total - F:
                wrap = iF + d >= inner
                out[d] = gF + d - (inner if wrap and not last_row else 0)
        return [out[d] for d in sorted(out)]
    m_inner, m_n = magic(inner), magic(n)
    one_slice = total == n * inner
    for t in range(256):
        a0 = iF + t
        assert a0 < (1 << 32)
        q = fastdiv(a0, m_inner)
        i = a0 - q * inner
        q256 = fastdiv(256, m_inner)
        r256 = 256 - q256 * inner
        for m in range(M):
            if m > 0:
                i += r256
                q += q256
                if i >= inner:
                    i -= inner
                    q += 1
            assert i < inner and jF + q < (1 << 32)
            b = 0 if one_slice else fastdiv(jF + q, m_n)
            d = m * 256 + t
            if d < total - F:
                out[d] = (oF + b) * inner + i
    return [out[d] for d in sorted(out)]


@pytest.mark.parametrize("K,U", [(4, 4), (8, 2), (1, 16)])
def test_flat_locate_matches_direct_index(K, U):
    CH = 256 * U * K
    rng = np.random.default_rng(K * 100 + U)
    shapes = [(1, 1, 2), (5, 1, 37), (7, 33, 12), (3, 5, 7), (2, 3000, 3), (1, 8192, 4096),
              (1, 3, CH + 1), (2, 3, CH - 1), (4, 2, 3 * CH + 5), (1, 2, 10 * CH + 3)]
    shapes += [(int(rng.integers(1, 6)), int(rng.integers(1, 50)), int(rng.integers(2, 3 * CH)))
               for _ in range(12)]
    for outer, n, inner in shapes:
        total = outer * n * inner
        starts = sorted({0, max(0, total - CH), *(int(v) for v in rng.integers(0, total, size=4))})
        for F in starts:
            got = locate_chunk(F, CH, n, inner, total)
            f = np.arange(F, F + len(got), dtype=np.int64)
            want = (f // (n * inner)) * inner + f % inner
            assert got == want.tolist(), (outer, n, inner, F)
