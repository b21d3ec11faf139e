"""Pins of the float64 oracle (CPU only).

The closed-form, brute-force and invariant checks live in ``oracle_pins.py``
so that the mutation test can run them on planted-mistake copies too. The
checks below add the library cross-check (SciPy) and closed forms taken from
the generators' own draws on prefixes of the five workloads.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle_pins
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

# Prefix sizes: each spans several of the GPU kernels' tiles and runs in well
# under a second through the oracle.
PREFIX = {1: 64, 2: 16, 3: 8, 4: 256, 5: 1 << 16}


@pytest.fixture(scope="module")
def prefixes():
    return {c: workloads.make(c, rows=n, aux=True) for c, n in PREFIX.items()}


@pytest.mark.parametrize("pin", oracle_pins.CHEAP_PINS, ids=lambda f: f.__name__)
def test_pin(oracle, pin):
    pin(oracle)


def _as_f64(w):
    if w.dtype == "bf16":
        return workloads.bf16_bits_to_f32(w.x).astype(np.float64)
    return w.x.astype(np.float64)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_scipy_logsumexp(oracle, prefixes, cfg):
    """A library routine: scipy.special.logsumexp in float64 on the same rows."""
    w = prefixes[cfg]
    got = oracle.lse(w.x, w.dtype, threads=4)
    want = scipy.special.logsumexp(_as_f64(w), axis=1)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin)
    assert np.all(got[~fin] == want[~fin])
    err = np.abs(got[fin] - want[fin]) / np.maximum(1.0, np.abs(want[fin]))
    assert err.max(initial=0.0) <= 1e-13


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_max_bounds(oracle, prefixes, cfg):
    """max_j x_j <= LSE <= max_j x_j + ln(#entries > -inf), on every row."""
    w = prefixes[cfg]
    got = oracle.lse(w.x, w.dtype, threads=4)
    x = _as_f64(w)
    mx = x.max(axis=1)
    count = np.isfinite(x).sum(axis=1)
    live = count > 0
    assert np.all(got[~live] == -np.inf)
    slack = 1e-12 * np.maximum(1.0, np.abs(mx[live]))
    assert np.all(got[live] >= mx[live] - slack)
    assert np.all(got[live] <= mx[live] + np.log(count[live]) + slack)


def test_config5_dirichlet_closed_form(oracle, prefixes):
    """x = fp32(ln p) with p a Dirichlet draw: LSE(x) = ln(sum of kept p_j).

    LSE is 1-Lipschitz in the max norm, so |LSE(x) - ln sum_kept p| is at most
    max_j |x_j - ln p_j| (the fp32 rounding of ln p), plus double rounding.
    Rows that keep every entry have sum p = 1, so their LSE is ~0.
    """
    w = prefixes[5]
    p, keep, allneg = w.aux["p"], w.aux["keep"].copy(), w.aux["allneg"]
    keep[allneg] = False
    got = oracle.lse(w.x, "f32", threads=4)
    mass = np.where(keep, p, 0.0).sum(axis=1)
    dead = ~keep.any(axis=1)
    assert np.all(got[dead] == -np.inf)
    assert dead.sum() >= len(allneg)
    lnp = np.log(p)
    delta = np.where(keep, np.abs(w.x.astype(np.float64) - lnp), 0.0).max(axis=1)
    live = ~dead
    err = np.abs(got[live] - np.log(mass[live]))
    assert np.all(err <= delta[live] + 4e-16 * np.maximum(1.0, np.abs(got[live])) + 1e-15)
    full = keep.all(axis=1)
    assert full.sum() > 1000
    assert np.all(np.abs(got[full]) <= delta[full] + 1e-15)


def test_config4_particle_rows_brute(oracle, prefixes):
    """Particle-filter rows: exact fsum brute force, and the closed-form mean.

    E[exp(-z^2/(2 s^2))] = s / sqrt(1 + s^2) for z ~ N(0, 1), so
    sum_j exp(x_ij) ~ 4096 / sqrt(1 + s_i^2) and LSE_i ~ ln 4096 - ln(1 + s_i^2)/2.
    """
    w = prefixes[4]
    got = oracle.lse(w.x, "f32", threads=4)
    for r in range(0, w.rows, 37):
        assert abs(got[r] - oracle_pins.brute_lse(w.x[r])) <= 1e-14 * max(1, abs(got[r]))
    sigma = w.aux["sigma"]
    pred = math.log(4096) - 0.5 * np.log1p(sigma * sigma)
    assert abs(np.mean(got - pred)) < 0.01
    assert np.percentile(np.abs(got - pred), 90) < 0.2


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_full_length_rows_brute_force(oracle, prefixes, cfg):
    """Whole rows of the long-row workloads (32000, 128256 and 262144
    elements) against log(fsum(exp(x))): every element decoded on its own
    (struct for bf16), summed exactly, no maximum subtracted. A term dropped,
    doubled or taken from the wrong place moves a row of N elements by about
    1/N relative, far above the bar; the oracle's own ascending double sum is
    within sqrt(N) ulps of the exact one."""
    w = prefixes[cfg]
    got = oracle.lse(w.x, w.dtype, threads=4)
    for r in sorted({0, w.rows // 2, w.rows - 1}):
        if w.dtype == "bf16":
            vals = [oracle_pins._bf16_value(b) for b in w.x[r].tolist()]
        else:
            vals = w.x[r].astype(np.float64).tolist()
        want = oracle_pins.brute_lse(vals)
        assert abs(got[r] - want) <= 1e-12 * max(1.0, abs(want)), (cfg, r, got[r], want)


def test_config2_spike_bound(oracle, prefixes):
    """Eight spike columns equal to bf16(o_i + 15) are the row maximum, so
    LSE_i >= spike + ln 8 and LSE_i <= spike + ln 8 + ln(1 + (N - 8) e^(next - spike) / 8)."""
    w = prefixes[2]
    got = oracle.lse(w.x, "bf16")
    x = _as_f64(w)
    spikes = w.aux["spikes"]
    for r in range(w.rows):
        sv = x[r, spikes[r]]
        assert np.all(sv == sv[0])
        rest = np.delete(x[r], spikes[r])
        assert rest.max() < sv[0]
        lo = sv[0] + math.log(8)
        hi = lo + math.log1p((x.shape[1] - 8) * math.exp(rest.max() - sv[0]) / 8)
        assert lo - 1e-12 <= got[r] <= hi + 1e-12


def test_prefix_rows_match_full_rows(oracle):
    """A prefix of a workload equals the same rows of a longer draw, bit for bit."""
    a = workloads.make(4, rows=1500)
    b = workloads.make(4, rows=1100)
    assert np.array_equal(a.x[:1100], b.x)


def test_golden_edge_cases(oracle):
    """The stored edge cases: the oracle reproduces them bit for bit, and every
    stored value agrees with brute-force summation where that cannot overflow."""
    import golden_cases
    cases = golden_cases.load()
    assert len(cases) >= 20
    for c in cases:
        got = oracle.lse(c["x"], c["dtype"])
        want = c["out"]
        assert np.array_equal(np.isnan(got), np.isnan(want)), c["name"]
        ok = ~np.isnan(want)
        assert np.array_equal(got[ok], want[ok]), c["name"]
        vals = c["x"] if c["dtype"] == "f32" else workloads.bf16_bits_to_f32(c["x"])
        for r in range(vals.shape[0]):
            row = vals[r].astype(np.float64)
            if np.all(np.abs(row[np.isfinite(row)]) < 700):
                w = oracle_pins.brute_lse(row)
                if np.isnan(w):
                    assert np.isnan(want[r]), c["name"]
                else:
                    assert abs(want[r] - w) <= 1e-14 * max(1.0, abs(w)) or want[r] == w, c["name"]


# --- LSE over a non-last axis --------------------------------------------

def test_lse_dim_against_scipy_and_brute_force(oracle):
    """The middle-axis oracle against scipy.special.logsumexp(axis=1) and, on
    tiny arrays, against log(fsum(exp)) of each gathered column."""
    from scipy.special import logsumexp
    import oracle as orc_mod
    rng = np.random.default_rng(30)
    for shape in [(1, 7, 5), (3, 1, 4), (2, 33, 17), (4, 100, 1), (1, 513, 64), (5, 2, 9)]:
        x = rng.normal(0, 6, size=shape).astype(np.float32)
        got = orc_mod.lse_dim(x, "f32")
        want = logsumexp(x.astype(np.float64), axis=1)
        assert got.shape == want.shape
        assert np.all(np.abs(got - want) <= 1e-13 * np.maximum(1.0, np.abs(want))), shape
        if x.size <= 2000:
            for o in range(shape[0]):
                for i in range(shape[2]):
                    w = oracle_pins.brute_lse(x[o, :, i])
                    assert abs(got[o, i] - w) <= 1e-14 * max(1.0, abs(w)), (shape, o, i)
    bits = workloads.f32_to_bf16_bits(rng.normal(0, 3, size=(3, 40, 11)).astype(np.float32))
    got = orc_mod.lse_dim(bits, "bf16")
    vals = workloads.bf16_bits_to_f32(bits).astype(np.float64)
    assert np.all(np.abs(got - logsumexp(vals, axis=1)) <= 1e-13 * np.maximum(1, np.abs(got)))
    # special columns: all -inf, a NaN, a +inf; and n = 0 gives -inf
    x = np.zeros((1, 4, 3), np.float32)
    x[0, :, 0] = -np.inf
    x[0, 2, 1] = np.nan
    x[0, 1, 2] = np.inf
    got = orc_mod.lse_dim(x, "f32")
    assert got[0, 0] == -np.inf and np.isnan(got[0, 1]) and got[0, 2] == np.inf
    assert np.all(orc_mod.lse_dim(np.zeros((2, 0, 3), np.float32), "f32") == -np.inf)


def test_lse_dim_grad_pins(oracle):
    """The middle-axis gradient oracle: (1) element by element against an
    explicit triple loop of g[o, i] * exp(x[o, j, i] - lse[o, i]) (math.exp,
    distinct values everywhere, so a transposed or shifted axis fails);
    (2) central finite differences of the brute-force (fsum) LSE of each
    column, weighted by g; (3) the column sums g * exp(LSE - lse32);
    (4) bf16 decoding and special values (NaN, -inf entries, an -inf column)."""
    import oracle as orc_mod
    rng = np.random.default_rng(31)
    # (1) explicit loop, with lse and g that are not the forward's
    x = rng.uniform(-3, 3, size=(2, 5, 3)).astype(np.float32)
    lse = rng.uniform(-1, 1, size=(2, 3)).astype(np.float32)
    g = rng.uniform(0.5, 2, size=(2, 3)).astype(np.float32)
    got = orc_mod.lse_dim_grad(x, lse, g, "f32")
    assert got.shape == x.shape
    for o in range(2):
        for j in range(5):
            for i in range(3):
                want = float(g[o, i]) * math.exp(float(x[o, j, i]) - float(lse[o, i]))
                assert abs(got[o, j, i] - want) <= 1e-14 * abs(want), (o, j, i)
    # (2) finite differences of sum_{o,i} g[o,i] * LSE(x)[o,i] with the fp32 LSE
    x = rng.uniform(-2, 2, size=(2, 4, 3)).astype(np.float64)
    g = rng.uniform(0.5, 2, size=(2, 3)).astype(np.float32)
    lse_exact = np.array([[oracle_pins.brute_lse(x[o, :, i]) for i in range(3)] for o in range(2)])
    got = orc_mod.lse_dim_grad(x.astype(np.float32), lse_exact.astype(np.float32), g, "f32")
    h = 1e-5
    for o in range(2):
        for j in range(4):
            for i in range(3):
                up, dn = x[o, :, i].copy(), x[o, :, i].copy()
                up[j] += h
                dn[j] -= h
                fd = float(g[o, i]) * (oracle_pins.brute_lse(up) - oracle_pins.brute_lse(dn)) / (2 * h)
                # the float32 inputs and lse differ from the float64 ones by < 1e-7 relative
                assert abs(got[o, j, i] - fd) <= 1e-6 * max(1.0, abs(fd)), (o, j, i, got[o, j, i], fd)
    # (3) column sums
    x = rng.normal(0, 3, size=(3, 50, 7)).astype(np.float32)
    lse32 = orc_mod.lse_dim(x, "f32").astype(np.float32)
    g = rng.normal(0, 1, size=(3, 7)).astype(np.float32)
    got = orc_mod.lse_dim_grad(x, lse32, g, "f32")
    exact = orc_mod.lse_dim(x, "f32")
    want = g.astype(np.float64) * np.exp(exact - lse32.astype(np.float64))
    assert np.all(np.abs(got.sum(axis=1) - want) <= 1e-12 * np.maximum(1.0, np.abs(want)))
    # (4) bf16 decoding, NaN and -inf entries, a column of -inf
    bits = workloads.f32_to_bf16_bits(rng.normal(0, 2, size=(1, 6, 4)).astype(np.float32))
    bits[0, 1, 0] = 0xFF80  # -inf entry
    bits[0, 2, 1] = 0x7FC0  # NaN entry
    bits[0, :, 3] = 0xFF80  # a column of -inf
    vals = workloads.bf16_bits_to_f32(bits).astype(np.float64)
    lse = np.zeros((1, 4), np.float32)
    lse[0, 3] = -np.inf
    g = np.ones((1, 4), np.float32)
    got = orc_mod.lse_dim_grad(bits, lse, g, "bf16")
    assert got[0, 1, 0] == 0.0
    assert np.isnan(got[0, 2, 1]) and np.isfinite(np.delete(got[0, :, 1], 2)).all()
    assert np.isnan(got[0, :, 3]).all()  # exp(-inf - (-inf)) is exp(NaN)
    mask = np.ones_like(vals, dtype=bool)
    mask[0, 1, 0] = mask[0, 2, 1] = False
    mask[0, :, 3] = False
    assert np.all(np.abs(got[mask] - np.exp(vals[mask])) <= 1e-14 * np.exp(vals[mask]))



# --- the oracle against 50-digit decimal arithmetic (hypothesis) ------------

import math  # noqa: E402
from decimal import Decimal, localcontext  # noqa: E402

from hypothesis import given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402


def decimal_lse(values) -> float:
    """log(sum(exp(v))) in 50-digit decimal arithmetic, which shares nothing
    with the oracle's libm exp/log: each float converts to Decimal exactly,
    -inf entries contribute nothing, and no exponent can overflow."""
    fin = [v for v in values if v != -math.inf]
    if not fin:
        return -math.inf
    with localcontext() as ctx:
        ctx.prec, ctx.Emax, ctx.Emin = 50, 10 ** 9, -10 ** 9
        m = Decimal(max(fin))
        total = sum((Decimal(v) - m).exp() for v in fin)
        return float(m + total.ln())


_F32 = st.floats(min_value=-2.0 ** 100, max_value=2.0 ** 100, width=32, allow_nan=False)
_ROW = st.lists(st.one_of(_F32, st.floats(-60, 60, width=32), st.just(-math.inf)),
                min_size=1, max_size=48)


@settings(max_examples=300, deadline=None)
@given(rows=st.lists(_ROW, min_size=1, max_size=6))
def test_oracle_matches_decimal_arithmetic_f32(oracle, rows):
    """Rows of mixed magnitudes (up to 2^100), clustered values and -inf."""
    width = max(len(r) for r in rows)
    x = np.full((len(rows), width), -np.inf, dtype=np.float32)
    for i, r in enumerate(rows):
        x[i, :len(r)] = r
    got = oracle.lse(x, "f32")
    for i in range(len(rows)):
        want = decimal_lse([float(v) for v in x[i]])
        if math.isinf(want):
            assert got[i] == want
        else:
            assert abs(got[i] - want) <= 1e-13 * max(1.0, abs(want)), (rows[i], got[i], want)


@settings(max_examples=200, deadline=None)
@given(bits=st.lists(st.lists(st.integers(0, 0xFFFF).filter(
    lambda b: (b & 0x7F80) != 0x7F80 or b == 0xFF80), min_size=1, max_size=40),
    min_size=1, max_size=4))
def test_oracle_matches_decimal_arithmetic_bf16(oracle, bits):
    """Every finite bf16 pattern (and -inf), decoded by placing the 16 bits
    high in an fp32 word, against the decimal reference."""
    width = max(len(r) for r in bits)
    x = np.full((len(bits), width), 0xFF80, dtype=np.uint16)
    for i, r in enumerate(bits):
        x[i, :len(r)] = r
    got = oracle.lse(x, "bf16")
    vals = (x.astype(np.uint32) << 16).view(np.float32)
    for i in range(len(bits)):
        want = decimal_lse([float(v) for v in vals[i]])
        if math.isinf(want):
            assert got[i] == want
        else:
            assert abs(got[i] - want) <= 1e-13 * max(1.0, abs(want)), (bits[i], got[i], want)


@settings(max_examples=200, deadline=None)
@given(bits=st.lists(st.lists(st.integers(0, 0xFFFF).filter(
    lambda b: (b & 0x7C00) != 0x7C00 or b == 0xFC00), min_size=1, max_size=40),
    min_size=1, max_size=4))
def test_oracle_matches_decimal_arithmetic_f16(oracle, bits):
    """Every finite fp16 pattern (and -inf), decoded by numpy's float16, against
    the decimal reference."""
    width = max(len(r) for r in bits)
    x = np.full((len(bits), width), 0xFC00, dtype=np.uint16)
    for i, r in enumerate(bits):
        x[i, :len(r)] = r
    got = oracle.lse(x, "f16")
    vals = x.view(np.float16).astype(np.float64)
    for i in range(len(bits)):
        want = decimal_lse([float(v) for v in vals[i]])
        if math.isinf(want):
            assert got[i] == want
        else:
            assert abs(got[i] - want) <= 1e-13 * max(1.0, abs(want)), (bits[i], got[i], want)
