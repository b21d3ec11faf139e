"""Checks that pin the float64 oracle to facts outside itself.

Each check takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with a closed form, a brute-force sum, a library routine or
an invariant of log-sum-exp. ``test_oracle.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes and expects each copy to fail at least one.

The expected values here never come from the oracle itself (nor from the HIP
library): they are written from the mathematics, in Python's own float64
arithmetic (``math.fsum``, ``math.log1p``, ``struct`` for bit decoding) or by
SciPy.
"""
from __future__ import annotations

import math
import struct

import numpy as np

LN2 = math.log(2.0)
LOG2E = 1.0 / LN2


def _close(got, want, rel=1e-14, what=""):
    got = float(got)
    want = float(want)
    if math.isnan(want):
        assert math.isnan(got), f"{what}: want NaN, got {got!r}"
        return
    if math.isinf(want):
        assert got == want, f"{what}: want {want!r}, got {got!r}"
        return
    tol = rel * max(1.0, abs(want))
    assert abs(got - want) <= tol, f"{what}: |{got!r} - {want!r}| > {tol:.3g}"


def _bf16_value(bits: int) -> float:
    """Decode a bf16 bit pattern with struct: high half of an fp32 word."""
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _f16_value(bits: int) -> float:
    """Decode an IEEE half bit pattern with struct's binary16 format."""
    return struct.unpack("<e", struct.pack("<H", int(bits) & 0xFFFF))[0]


def brute_lse(values) -> float:
    """log(sum exp(v)) by exact summation; only for |v| small enough not to overflow."""
    vals = [float(v) for v in values]
    if any(math.isnan(v) for v in vals):
        return math.nan
    if not vals or all(v == -math.inf for v in vals):
        return -math.inf
    if any(v == math.inf for v in vals):
        return math.inf
    return math.log(math.fsum(math.exp(v) for v in vals if v != -math.inf))


def pair_lse(a: float, b: float) -> float:
    """The pairwise operator in the base-2 form f(z) = log2(1 + 2^z), z <= 0.

    The paper's IntLSE error analysis (§A.1) takes f(z) = log2(1 + 2^z) as the
    exact pairwise correction: lse(a, b) = ln 2 * (max' + f(min' - max')) with
    a' = a * log2(e). Written here with log1p/exp2 in float64.
    """
    hi, lo = max(a, b), min(a, b)
    if hi == -math.inf:
        return -math.inf
    z = (lo - hi) * LOG2E          # z <= 0, in base-2 units
    # ln 2 * f(z) = ln 2 * log2(1 + 2^z) = log1p(2^z)
    return hi + math.log1p(2.0 ** z)


# --- closed forms --------------------------------------------------------

def pin_constant_rows(orc):
    """A row of N copies of c gives c + ln N (sum of N ones, exactly N)."""
    for c in (0.0, 1.5, -7.25, 100.0, 800.0, -800.0, -29952.0):
        for n in (1, 2, 3, 7, 1000, 32000):
            x = np.full((2, n), c, dtype=np.float32)
            got = orc.lse(x, "f32")
            _close(got[0], c + math.log(n), 4e-16, f"f32 const c={c} N={n}")
            _close(got[1], c + math.log(n), 4e-16, f"f32 const c={c} N={n} (row 1)")
            # the same constant as bf16 (every c above is a bf16 value)
            bits = np.full((1, n), struct.unpack("<I", struct.pack("<f", c))[0] >> 16,
                           dtype=np.uint16)
            _close(orc.lse(bits, "bf16")[0], c + math.log(n), 4e-16, f"bf16 const c={c} N={n}")


def pin_two_element_closed_form(orc):
    """Two-element rows against the base-2 pairwise form f(z) (§A.1)."""
    rng = np.random.default_rng(11)
    pairs = [(0.0, 0.0), (1.0, 0.0), (0.0, 1.0), (800.0, 0.0), (0.0, -800.0),
             (-1000.0, 1000.0), (3.5, -2.25), (-60.0, -61.0), (30.0, -60.0)]
    pairs += [tuple(v) for v in rng.uniform(-40, 40, size=(40, 2)).astype(np.float32)]
    x = np.array(pairs, dtype=np.float32)
    got = orc.lse(x, "f32")
    for (a, b), g in zip(x.astype(np.float64), got):
        _close(g, pair_lse(a, b), 1e-14, f"pair ({a}, {b})")


def pin_brute_force_tiny(orc):
    """Rows of <= 64 elements with |x| <= 50 against log(fsum(exp(x))), strided."""
    rng = np.random.default_rng(5)
    for cols in (1, 2, 3, 5, 8, 16, 17, 33, 64):
        for stride in (cols, cols + 3):
            buf = rng.uniform(-50, 50, size=(6, stride)).astype(np.float32)
            view = buf[:, :cols]
            got = orc.lse(view, "f32")
            for r in range(view.shape[0]):
                _close(got[r], brute_lse(view[r]), 1e-14, f"f32 brute cols={cols} r={r}")
            bits = (rng.integers(0, 1 << 16, size=(5, stride), dtype=np.uint32)).astype(np.uint16)
            # keep finite values with |x| <= 50: clear exponents above 2^5
            vals = [[_bf16_value(b) for b in row] for row in bits]
            for r in range(bits.shape[0]):
                for j in range(stride):
                    if not math.isfinite(vals[r][j]) or abs(vals[r][j]) > 50:
                        bits[r, j] = 0x3F80 if j % 2 else 0xC1A0  # 1.0 or -20.0
            bview = bits[:, :cols]
            got = orc.lse(bview, "bf16")
            for r in range(bview.shape[0]):
                want = brute_lse([_bf16_value(b) for b in bview[r]])
                _close(got[r], want, 1e-14, f"bf16 brute cols={cols} r={r}")


def pin_special_values(orc):
    """NaN, +-inf, empty and subnormal rows (semantics of torch.logsumexp)."""
    inf, nan = math.inf, math.nan
    cases = [
        ([-inf, -inf, -inf], -inf),
        ([-inf], -inf),
        ([1.0, nan, 2.0], nan),
        ([nan, 1.0], nan),
        ([inf, 1.0, -inf], inf),
        ([1.0, inf], inf),
        ([inf, nan], nan),
        ([nan, inf], nan),
        ([-inf, nan], nan),
        ([-inf, 0.0], 0.0),
        ([0.0, -inf, -inf, 0.0], LN2),
        ([1e-45, -inf], 1e-45),
        ([3.0e38, 3.0e38], None),
        ([-3.0e38, -3.0e38, -3.0e38], None),
    ]
    for row, want in cases:
        x = np.array([row], dtype=np.float32)
        if want is None:  # huge magnitudes: m + ln(count)
            v = float(x[0, 0])
            want = v + math.log(len(row))
        elif want == 1e-45:
            want = float(np.float32(1e-45))
        _close(orc.lse(x, "f32")[0], want, 1e-15, f"special {row}")
    # empty rows: the empty sum gives -inf
    got = orc.lse(np.zeros((3, 0), dtype=np.float32), "f32")
    assert np.all(got == -np.inf), f"cols=0 gave {got}"
    # bf16 specials: 0x7F80 = +inf, 0xFF80 = -inf, 0x7FC1 = NaN
    b = np.array([[0xFF80, 0xFF80], [0x7F80, 0x3F80], [0x7FC1, 0x3F80], [0x3F80, 0x3F80]],
                 dtype=np.uint16)
    got = orc.lse(b, "bf16")
    assert got[0] == -np.inf and got[1] == np.inf and np.isnan(got[2]), f"bf16 specials {got}"
    _close(got[3], 1.0 + LN2, 1e-15, "bf16 [1, 1]")


# --- fp16 inputs (the 16-bit reading of the paper's FuseLSE16, §4.3) ----------

def pin_f16_every_pattern(orc):
    """All 65536 fp16 bit patterns as one-element rows: the LSE of a single
    element is the element, so every decoded value is checked exactly against
    struct's binary16 decoding (NaN patterns give NaN, +-inf themselves)."""
    bits = np.arange(1 << 16, dtype=np.uint16).reshape(-1, 1)
    got = orc.lse(bits, "f16")
    for b in range(1 << 16):
        want = _f16_value(b)
        if math.isnan(want):
            assert math.isnan(got[b]), f"f16 pattern {b:#06x}: want NaN, got {got[b]!r}"
        else:
            assert got[b] == want, f"f16 pattern {b:#06x}: want {want!r}, got {got[b]!r}"


def pin_f16_rows(orc):
    """fp16 rows (strided, random finite patterns with |x| <= 50, and special
    rows) against log(fsum(exp)) of struct-decoded values; constant rows
    c + ln N; and the token log-probability and softmax gradient of fp16 rows
    against the same brute force."""
    rng = np.random.default_rng(21)
    for cols in (1, 3, 8, 17, 64):
        for stride in (cols, cols + 5):
            bits = rng.integers(0, 1 << 16, size=(6, stride), dtype=np.uint32).astype(np.uint16)
            vals = [[_f16_value(b) for b in row] for row in bits]
            for r in range(bits.shape[0]):
                for j in range(stride):
                    if not math.isfinite(vals[r][j]) or abs(vals[r][j]) > 50:
                        bits[r, j] = 0x3C00 if j % 2 else 0xCD00  # 1.0 or -20.0
            view = bits[:, :cols]
            got = orc.lse(view, "f16")
            for r in range(view.shape[0]):
                want = brute_lse([_f16_value(b) for b in view[r]])
                _close(got[r], want, 1e-14, f"f16 brute cols={cols} r={r}")
            t = rng.integers(0, cols, size=view.shape[0])
            got = orc.token_logprob(view, t, "f16")
            for r in range(view.shape[0]):
                v = [_f16_value(b) for b in view[r]]
                bl = brute_lse(v)
                _close(got[r], v[t[r]] - bl, 1e-14 * max(1.0, abs(bl)) / max(1.0, abs(v[t[r]] - bl)),
                       f"f16 logprob cols={cols} r={r}")
    for c, h in ((1.0, 0x3C00), (-20.0, 0xCD00), (65504.0, 0x7BFF), (2.0 ** -24, 0x0001)):
        for n in (1, 7, 1000):
            row = np.full((1, n), h, dtype=np.uint16)
            _close(orc.lse(row, "f16")[0], c + math.log(n), 4e-16, f"f16 const c={c} N={n}")
    # specials: 0x7C00 = +inf, 0xFC00 = -inf, 0x7E00 = NaN
    b = np.array([[0xFC00, 0xFC00], [0x7C00, 0x3C00], [0x7E00, 0x3C00], [0x3C00, 0x3C00]],
                 dtype=np.uint16)
    got = orc.lse(b, "f16")
    assert got[0] == -np.inf and got[1] == np.inf and np.isnan(got[2]), f"f16 specials {got}"
    _close(got[3], 1.0 + LN2, 1e-15, "f16 [1, 1]")
    # the softmax gradient of fp16 rows: exp(x - lse) with struct-decoded x
    bits = np.array([[0x3C00, 0xBC00, 0x4000, 0x0000, 0x0001]], dtype=np.uint16)
    v = [_f16_value(b) for b in bits[0]]
    lse32 = np.array([brute_lse(v)], dtype=np.float32)
    got = orc.softmax_grad(bits, lse32, np.array([2.0], np.float32), "f16")
    for j in range(5):
        want = 2.0 * math.exp(v[j] - float(lse32[0]))
        assert abs(got[0, j] - want) <= 1e-15 * max(1.0, want), f"f16 grad j={j}"


# --- invariants --------------------------------------------------------------

def pin_shift_invariance(orc):
    """LSE(x + c) = LSE(x) + c, with x on a 1/64 grid so x + c is exact in fp32."""
    rng = np.random.default_rng(7)
    x = (rng.integers(-640, 640, size=(8, 300)) / 64.0).astype(np.float32)
    base = orc.lse(x, "f32")
    for k in (-3, 0, 4, 7):
        c = np.float32(2.0 ** k)
        shifted = orc.lse(x + c, "f32")
        for r in range(x.shape[0]):
            _close(shifted[r], base[r] + float(c), 1e-14, f"shift 2^{k} r={r}")


def pin_permutation_invariance(orc):
    """The pairwise operator is commutative (§3.1): any column order, same value."""
    rng = np.random.default_rng(8)
    x = rng.normal(0, 5, size=(6, 513)).astype(np.float32)
    base = orc.lse(x, "f32")
    for _ in range(3):
        perm = rng.permutation(x.shape[1])
        _close_all(orc.lse(np.ascontiguousarray(x[:, perm]), "f32"), base, 1e-14, "permutation")


def pin_concat_merge(orc):
    """Associativity (§3.1): LSE(a ++ b) = lse(LSE(a), LSE(b)) via the pairwise form."""
    rng = np.random.default_rng(9)
    a = rng.normal(0, 4, size=(5, 200)).astype(np.float32)
    b = (rng.normal(0, 4, size=(5, 77)) + 9).astype(np.float32)
    whole = orc.lse(np.concatenate([a, b], axis=1), "f32")
    la, lb = orc.lse(a, "f32"), orc.lse(b, "f32")
    for r in range(a.shape[0]):
        _close(whole[r], pair_lse(la[r], lb[r]), 1e-14, f"concat r={r}")


def pin_thread_count_invariance(orc):
    """The row split over threads changes nothing, bit for bit."""
    rng = np.random.default_rng(10)
    for rows in (1, 2, 7, 10, 33):
        x = rng.normal(0, 3, size=(rows, 45)).astype(np.float32)
        one = orc.lse(x, "f32", threads=1)
        for t in (2, 3, 7, 64):
            assert np.array_equal(orc.lse(x, "f32", threads=t), one), f"threads={t} rows={rows}"
        for r in range(rows):
            _close(one[r], brute_lse(x[r]), 1e-14, f"threads brute r={r}")


def pin_argument_checks(orc):
    out = np.empty(4)
    x = np.zeros((4, 4), np.float32)
    assert orc.raw(x.ctypes.data, 3, 4, 4, 4, out.ctypes.data) == -1, "bad dtype accepted"
    assert orc.raw(x.ctypes.data, 0, -1, 4, 4, out.ctypes.data) == -1, "rows < 0 accepted"
    assert orc.raw(x.ctypes.data, 0, 4, -1, 4, out.ctypes.data) == -1, "cols < 0 accepted"
    assert orc.raw(x.ctypes.data, 0, 4, 4, 3, out.ctypes.data) == -1, "stride < cols accepted"
    assert orc.raw(None, 0, 0, 4, 4, None) == 0, "rows = 0 must be a no-op"
    assert orc.raw(None, 0, 4, 4, 4, out.ctypes.data) == -1, "null x accepted"


# --- token log-probabilities ---------------------------------------------
#
# logp = x[t] - LSE(x): the log-probability of column t under a softmax over
# the row, the per-token quantity the paper's RLHF workload computes (§1, §5.1).

def _close_logp(got, want, scale, what):
    """|got - want| <= 1e-14 * max(1, |scale|): logp inherits the LSE's error."""
    got, want = float(got), float(want)
    if math.isnan(want) or math.isinf(want):
        _close(got, want, 0.0, what)
        return
    tol = 1e-14 * max(1.0, abs(scale))
    assert abs(got - want) <= tol, f"{what}: |{got!r} - {want!r}| > {tol:.3g}"


def pin_logprob_softmax_normalised(orc):
    """exp(logp) summed over every target of a row is 1: a softmax is a distribution."""
    rng = np.random.default_rng(12)
    for cols in (1, 2, 3, 7, 33, 100):
        for r in range(3):
            row = rng.normal(0, 4, size=cols).astype(np.float32)
            copies = np.repeat(row[None, :], cols, axis=0)   # copy j asks for column j
            lp = orc.token_logprob(copies, np.arange(cols), "f32")
            s = math.fsum(math.exp(v) for v in lp)
            assert abs(s - 1.0) <= 1e-13 * cols, f"softmax over cols={cols} sums to {s!r}"
            # and the largest element has the largest log-probability
            assert int(np.argmax(lp)) == int(np.argmax(row)), f"argmax cols={cols}"


def pin_logprob_two_elements(orc):
    """Two-element rows: logp(t) = x_t - lse(a, b) in the base-2 pairwise form (§A.1)."""
    rng = np.random.default_rng(13)
    pairs = [(0.0, 0.0), (1.0, 0.0), (0.0, 1.0), (800.0, 0.0), (-1000.0, 1000.0),
             (3.5, -2.25), (-60.0, -61.0)]
    pairs += [tuple(v) for v in rng.uniform(-40, 40, size=(30, 2)).astype(np.float32)]
    x = np.array(pairs, dtype=np.float32)
    for t in (0, 1):
        got = orc.token_logprob(x, np.full(len(pairs), t), "f32")
        for (a, b), g in zip(x.astype(np.float64), got):
            pl = pair_lse(a, b)
            _close_logp(g, (a, b)[t] - pl, pl, f"pair ({a}, {b}) t={t}")


def pin_logprob_constant_rows(orc):
    """A row of N copies of c gives -ln N for every target, whatever c."""
    for c in (0.0, -7.25, 800.0, -800.0):
        for n in (1, 2, 7, 1000):
            x = np.full((3, n), c, dtype=np.float32)
            got = orc.token_logprob(x, [0, n // 2, n - 1], "f32")
            for g in got:
                _close_logp(g, -math.log(n), c + math.log(n), f"const c={c} N={n}")


def pin_logprob_brute_force(orc):
    """Tiny strided rows, fp32 and bf16 (decoded with struct), against x_t - log(fsum(exp))."""
    rng = np.random.default_rng(14)
    for cols in (1, 2, 5, 16, 33):
        buf = rng.uniform(-50, 50, size=(6, cols + 3)).astype(np.float32)
        view = buf[:, :cols]
        t = rng.integers(0, cols, size=6)
        got = orc.token_logprob(view, t, "f32")
        for r in range(6):
            bl = brute_lse(view[r])
            _close_logp(got[r], float(view[r, t[r]]) - bl, bl, f"f32 brute cols={cols} r={r}")
        bits = rng.integers(0x3F00, 0x4248, size=(6, cols + 3)).astype(np.uint16)  # 0.5 .. 50
        bits[::2] |= 0x8000                                                       # some negatives
        bview = bits[:, :cols]
        got = orc.token_logprob(bview, t, "bf16")
        for r in range(6):
            vals = [_bf16_value(b) for b in bview[r]]
            bl = brute_lse(vals)
            _close_logp(got[r], vals[t[r]] - bl, bl, f"bf16 brute cols={cols} r={r}")


def pin_logprob_special_values(orc):
    """IEEE arithmetic on x_t - LSE, and NaN for a target outside the row."""
    inf, nan = math.inf, math.nan
    cases = [
        ([-inf, 0.0, 1.0], 0, -inf),        # target at -inf
        ([-inf, -inf], 1, nan),            # -inf - -inf
        ([inf, 0.0], 1, -inf),             # +inf elsewhere
        ([inf, 0.0], 0, nan),              # +inf at the target: inf - inf
        ([nan, 0.0], 1, nan),
        ([0.0, 0.0], -1, nan),             # targets out of range
        ([0.0, 0.0], 2, nan),
        ([0.0, 0.0], 1 << 40, nan),
        ([0.0, -inf], 0, 0.0),             # a single finite element: probability 1
    ]
    for row, t, want in cases:
        x = np.array([row], dtype=np.float32)
        _close(orc.token_logprob(x, [t], "f32")[0], want, 1e-15, f"special {row} t={t}")
    got = orc.token_logprob(np.zeros((2, 0), dtype=np.float32), [0, -1], "f32")
    assert np.all(np.isnan(got)), f"cols=0 gave {got}"


def pin_logprob_shift_invariance(orc):
    """A softmax is invariant to adding c to the row (x on a 1/64 grid: exact in fp32)."""
    rng = np.random.default_rng(15)
    x = (rng.integers(-640, 640, size=(8, 300)) / 64.0).astype(np.float32)
    t = rng.integers(0, 300, size=8)
    base = orc.token_logprob(x, t, "f32")
    lse = orc.lse(x, "f32")
    for k in (-3, 4, 7):
        shifted = orc.token_logprob(x + np.float32(2.0 ** k), t, "f32")
        for r in range(8):
            _close_logp(shifted[r], base[r], lse[r] + 2.0 ** k, f"logp shift 2^{k} r={r}")


def pin_logprob_argument_checks(orc):
    x = np.zeros((4, 4), np.float32)
    out = np.empty(4)
    fn = orc._fn_tok
    assert fn(x.ctypes.data, 0, 4, 4, 4, None, out.ctypes.data, 1) == -1, "null targets accepted"
    t = np.zeros(4, np.int64)
    assert fn(x.ctypes.data, 0, 4, 4, 3, t.ctypes.data, out.ctypes.data, 1) == -1, \
        "stride < cols accepted"
    assert fn(None, 0, 0, 4, 4, None, None, 1) == 0, "rows = 0 must be a no-op"


# --- backward: the gradient of LSE ---------------------------------------
#
# d LSE(x) / d x_j = exp(x_j - LSE(x)), the row's softmax (backward support,
# Table 3). The oracle takes the forward value as fp32 (lse32), so the exact
# result is g * exp(x_j - L) * exp(L - lse32) with L the exact LSE; the
# factor exp(L - lse32) is computed here from the brute-force L.

def _fd_softmax(vals, j, h=1e-4):
    """d LSE / d x_j by a central difference of the brute-force LSE."""
    up = list(vals)
    dn = list(vals)
    up[j] += h
    dn[j] -= h
    return (brute_lse(up) - brute_lse(dn)) / (2 * h)


def pin_grad_finite_difference(orc):
    """The backward pass is the derivative of LSE: central differences of the
    brute-force LSE, element by element, and the softmax sums to one."""
    rng = np.random.default_rng(16)
    for cols in (1, 2, 3, 7, 20):
        x = rng.uniform(-20, 20, size=(4, cols + 2)).astype(np.float32)[:, :cols]
        vals = [[float(v) for v in row] for row in x]
        exact = [brute_lse(v) for v in vals]
        lse32 = np.array(exact, dtype=np.float32)
        g = np.array([1.0, -2.5, 0.125, 3.0], dtype=np.float32)
        got = orc.softmax_grad(x, lse32, g, "f32")
        for r in range(4):
            corr = math.exp(exact[r] - float(lse32[r]))
            for j in range(cols):
                want = float(g[r]) * _fd_softmax(vals[r], j) * corr
                assert abs(got[r, j] - want) <= 1e-7 * abs(float(g[r])) + 1e-7 * abs(want), \
                    f"finite difference r={r} j={j}: {got[r, j]!r} vs {want!r}"
            s = math.fsum(got[r])
            assert abs(s - float(g[r]) * corr) <= 1e-13 * max(1.0, abs(float(g[r]))), \
                f"softmax sum r={r}: {s!r}"


def pin_grad_two_elements(orc):
    """Two-element rows: the softmax of (a, b) against the base-2 pairwise form (§A.1)."""
    rng = np.random.default_rng(17)
    x = rng.uniform(-30, 30, size=(20, 2)).astype(np.float32)
    pl = [pair_lse(float(a), float(b)) for a, b in x]
    lse32 = np.array(pl, dtype=np.float32)
    g = np.full(20, 1.5, dtype=np.float32)
    got = orc.softmax_grad(x, lse32, g, "f32")
    for r in range(20):
        for j in range(2):
            want = 1.5 * math.exp(float(x[r, j]) - pl[r]) * math.exp(pl[r] - float(lse32[r]))
            _close(got[r, j], want, 1e-14, f"pair grad r={r} j={j}")


def pin_grad_constant_rows(orc):
    """A constant row of N gives g / N in every column (with lse = c + ln N exactly)."""
    for n in (1, 2, 4, 64, 1024):
        c = 3.0
        lse = c + math.log(n)
        x = np.full((2, n), c, dtype=np.float32)
        lse32 = np.full(2, lse, dtype=np.float32)
        got = orc.softmax_grad(x, lse32, [2.0, -1.0], "f32")
        corr = math.exp(lse - float(lse32[0]))
        for r, g in enumerate((2.0, -1.0)):
            for j in (0, n - 1):
                _close(got[r, j], g / n * corr, 1e-14, f"const grad N={n}")


def pin_grad_brute_force_bf16(orc):
    """bf16 rows decoded with struct, against fsum-based LSE and exp."""
    rng = np.random.default_rng(18)
    bits = rng.integers(0x3F00, 0x4200, size=(5, 9)).astype(np.uint16)   # 0.5 .. 32
    bits[1::2] |= 0x8000
    vals = [[_bf16_value(b) for b in row] for row in bits]
    exact = [brute_lse(v) for v in vals]
    lse32 = np.array(exact, dtype=np.float32)
    got = orc.softmax_grad(bits, lse32, np.ones(5, np.float32), "bf16")
    for r in range(5):
        corr = math.exp(exact[r] - float(lse32[r]))
        for j in range(9):
            want = _fd_softmax(vals[r], j) * corr
            assert abs(got[r, j] - want) <= 1e-7 * (1 + abs(want)), f"bf16 grad r={r} j={j}"


def pin_grad_special_values(orc):
    """IEEE arithmetic on grad_out * exp(x - lse)."""
    inf, nan = math.inf, math.nan
    x = np.array([[-inf, -inf], [-inf, 0.0], [inf, 0.0], [nan, 0.0], [1.0, 2.0]],
                 dtype=np.float32)
    lse = np.array([-inf, 0.0, inf, nan, 0.0], dtype=np.float32)
    g = np.array([1.0, 1.0, 1.0, 1.0, 0.0], dtype=np.float32)
    got = orc.softmax_grad(x, lse, g, "f32")
    assert np.isnan(got[0]).all(), "all -inf row: -inf - -inf"
    assert got[1, 0] == 0.0 and got[1, 1] == 1.0, "a -inf element gets 0"
    assert np.isnan(got[2, 0]) and got[2, 1] == 0.0, "+inf at lse +inf: NaN and 0"
    assert np.isnan(got[3]).all(), "NaN lse"
    assert np.all(got[4] == 0.0), "zero incoming gradient"
    got = orc.softmax_grad(np.zeros((3, 0), np.float32), np.zeros(3), np.ones(3), "f32")
    assert got.shape == (3, 0)


def pin_grad_argument_checks(orc):
    x = np.zeros((4, 4), np.float32)
    out = np.empty((4, 4))
    lse = np.zeros(4, np.float32)
    fn = orc._fn_grad
    assert fn(x.ctypes.data, 0, 4, 4, 4, None, lse.ctypes.data, out.ctypes.data, 1) == -1
    assert fn(x.ctypes.data, 0, 4, 4, 4, lse.ctypes.data, None, out.ctypes.data, 1) == -1
    assert fn(x.ctypes.data, 0, 4, 4, 3, lse.ctypes.data, lse.ctypes.data, out.ctypes.data, 1) == -1


# --- backward of the token log-probability ----------------------------------
# logp = x_t - LSE(x) has derivative [j == t] - softmax_j. The oracle takes the
# forward LSE as fp32 (lse32), so its exact result is
# g * ([j == t] - softmax_j * exp(L - lse32)) with L the exact LSE.

def _logp(vals, t):
    return vals[t] - brute_lse(vals)


def _fd_logp(vals, t, j, h=1e-4):
    up = list(vals)
    dn = list(vals)
    up[j] += h
    dn[j] -= h
    return (_logp(up, t) - _logp(dn, t)) / (2 * h)


def pin_tokgrad_finite_difference(orc):
    """Central differences of the brute-force log-probability, element by element."""
    rng = np.random.default_rng(30)
    for cols in (1, 2, 5, 16):
        x = rng.uniform(-15, 15, size=(4, cols + 3)).astype(np.float32)[:, :cols]  # padded rows
        t = rng.integers(0, cols, size=4)
        vals = [[float(v) for v in row] for row in x]
        exact = [brute_lse(v) for v in vals]
        lse32 = np.array(exact, dtype=np.float32)
        g = np.array([1.0, -3.0, 0.25, 2.0], dtype=np.float32)
        got = orc.token_logprob_grad(x, t, lse32, g, "f32")
        for r in range(4):
            corr = math.exp(exact[r] - float(lse32[r]))
            for j in range(cols):
                fd = _fd_logp(vals[r], int(t[r]), j)          # [j == t] - softmax_j
                delta = 1.0 if j == t[r] else 0.0
                want = float(g[r]) * (delta - (delta - fd) * corr)
                assert abs(got[r, j] - want) <= 1e-7 * max(1.0, abs(float(g[r]))), \
                    f"token grad finite difference r={r} j={j}: {got[r, j]!r} vs {want!r}"


def pin_tokgrad_row_sums(orc):
    """The one-hot term and the softmax each sum to one: a row sums to
    g * (1 - exp(L - lse32))."""
    rng = np.random.default_rng(31)
    x = rng.normal(0, 4, size=(6, 300)).astype(np.float32)
    t = rng.integers(0, 300, size=6)
    exact = [brute_lse([float(v) for v in row]) for row in x]
    lse32 = np.array(exact, dtype=np.float32)
    g = rng.normal(0, 2, size=6).astype(np.float32)
    got = orc.token_logprob_grad(x, t, lse32, g, "f32")
    for r in range(6):
        want = float(g[r]) * (1.0 - math.exp(exact[r] - float(lse32[r])))
        assert abs(math.fsum(got[r]) - want) <= 1e-12 * max(1.0, abs(float(g[r]))), f"row sum r={r}"


def pin_tokgrad_two_elements(orc):
    """Rows (a, b): the softmax of column 0 is 1 / (1 + e^(b - a))."""
    rng = np.random.default_rng(32)
    x = rng.uniform(-20, 20, size=(12, 2)).astype(np.float32)
    t = np.array([0, 1] * 6)
    pl = [pair_lse(float(a), float(b)) for a, b in x]
    lse32 = np.array(pl, dtype=np.float32)
    g = np.full(12, -0.75, dtype=np.float32)
    got = orc.token_logprob_grad(x, t, lse32, g, "f32")
    for r in range(12):
        a, b = float(x[r, 0]), float(x[r, 1])
        p0 = 1.0 / (1.0 + math.exp(b - a))
        corr = math.exp(pl[r] - float(lse32[r]))
        p = (p0 * corr, (1.0 - p0) * corr)
        for j in range(2):
            want = -0.75 * ((1.0 if j == t[r] else 0.0) - p[j])
            assert abs(got[r, j] - want) <= 1e-13, f"pair token grad r={r} j={j}"


def pin_tokgrad_targets(orc):
    """A target outside [0, cols) gives a row of NaN; other rows are untouched."""
    x = np.zeros((4, 5), dtype=np.float32)
    lse32 = np.full(4, math.log(5.0), dtype=np.float32)
    got = orc.token_logprob_grad(x, [-1, 5, 2, 1 << 40], lse32, np.ones(4, np.float32), "f32")
    assert np.isnan(got[0]).all() and np.isnan(got[1]).all() and np.isnan(got[3]).all()
    corr = math.exp(math.log(5.0) - float(lse32[2]))
    for j in range(5):
        _close(got[2, j], (1.0 if j == 2 else 0.0) - 0.2 * corr, 1e-14, f"target row j={j}")


def pin_tokgrad_argument_checks(orc):
    x = np.zeros((4, 4), np.float32)
    out = np.empty((4, 4))
    v = np.zeros(4, np.float32)
    t = np.zeros(4, np.int64)
    fn = orc._fn_tok_grad
    assert fn(x.ctypes.data, 0, 4, 4, 4, None, v.ctypes.data, v.ctypes.data, out.ctypes.data, 1) == -1
    assert fn(x.ctypes.data, 0, 4, 4, 4, t.ctypes.data, None, v.ctypes.data, out.ctypes.data, 1) == -1
    assert fn(x.ctypes.data, 0, 4, 4, 4, t.ctypes.data, v.ctypes.data, None, out.ctypes.data, 1) == -1


def _close_all(got, want, rel, what):
    assert got.shape == want.shape, f"{what}: shape"
    for i, (g, w) in enumerate(zip(got, want)):
        _close(g, w, rel, f"{what}[{i}]")


CHEAP_PINS = [
    pin_tokgrad_argument_checks,
    pin_tokgrad_finite_difference,
    pin_tokgrad_row_sums,
    pin_tokgrad_two_elements,
    pin_tokgrad_targets,
    pin_argument_checks,
    pin_constant_rows,
    pin_two_element_closed_form,
    pin_special_values,
    pin_brute_force_tiny,
    pin_shift_invariance,
    pin_permutation_invariance,
    pin_concat_merge,
    pin_thread_count_invariance,
    pin_logprob_argument_checks,
    pin_logprob_softmax_normalised,
    pin_logprob_two_elements,
    pin_logprob_constant_rows,
    pin_logprob_brute_force,
    pin_logprob_special_values,
    pin_logprob_shift_invariance,
    pin_grad_argument_checks,
    pin_grad_finite_difference,
    pin_grad_two_elements,
    pin_grad_constant_rows,
    pin_grad_brute_force_bf16,
    pin_grad_special_values,
    pin_f16_every_pattern,
    pin_f16_rows,
]
