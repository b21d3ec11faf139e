"""The seeded generators produce the stated shapes and distributions (CPU only)."""
import struct

import numpy as np
import pytest

import workloads


def test_specs_match_stated_sizes():
    s = workloads.SPECS
    assert (s[1].dtype, s[1].rows, s[1].cols) == ("f32", 64, 32000)
    assert (s[2].dtype, s[2].rows, s[2].cols) == ("bf16", 512, 128256)
    assert (s[3].dtype, s[3].rows, s[3].cols) == ("bf16", 4096, 262144)
    assert (s[4].dtype, s[4].rows, s[4].cols) == ("f32", 65536, 4096)
    assert (s[5].dtype, s[5].rows, s[5].cols) == ("f32", 1 << 24, 16)


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -3.3e38, 3.4e38,
                     np.inf, -np.inf, 0.0, -0.0, 1e-40], dtype=np.float32)
    got = workloads.f32_to_bf16_bits(vals)
    for v, b in zip(vals, got):
        u = struct.unpack("<I", struct.pack("<f", float(v)))[0]
        lo = u & 0xFFFF
        hi = u >> 16
        if lo > 0x8000 or (lo == 0x8000 and hi & 1):
            hi += 1
        assert int(b) == hi & 0xFFFF, (v, hex(int(b)), hex(hi))
    assert np.array_equal(workloads.bf16_bits_to_f32(got[:4]),
                          np.array([1.0, 1.0, 1.0078125, 1.0078125], np.float32))


def test_config1_is_deterministic_and_normal():
    a = workloads.make(1)
    b = workloads.make(1)
    assert a.x.dtype == np.float32 and a.x.shape == (64, 32000)
    assert workloads.sha256(a.x) == workloads.sha256(b.x)
    assert abs(a.x.mean()) < 0.01 and abs(a.x.std() - 3.0) < 0.01


def test_config2_offsets_and_spikes():
    w = workloads.make(2, rows=64, aux=True)
    assert w.x.dtype == np.uint16 and w.x.shape == (64, 128256)
    x = workloads.bf16_bits_to_f32(w.x)
    off = w.aux["offset"]
    assert np.all((off >= -20) & (off <= 20))
    spikes = w.aux["spikes"]
    assert all(len(set(r)) == 8 for r in spikes)
    want = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.float32(15.0) + off))
    assert np.array_equal(x[np.arange(64), spikes[:, 0]], want)
    body = x - off[:, None].astype(np.float32)
    mask = np.ones_like(x, dtype=bool)
    mask[np.arange(64)[:, None], spikes] = False
    assert abs(body[mask].std() - 2.0) < 0.05


def test_config3_neginf_fraction():
    w = workloads.make(3, rows=8)
    x = workloads.bf16_bits_to_f32(w.x)
    frac = np.isneginf(x).mean()
    assert 0.009 < frac < 0.011
    assert abs(x[np.isfinite(x)].std() - 4.0) < 0.02


def test_config4_rows():
    w = workloads.make(4, rows=512, aux=True)
    sig = w.aux["sigma"]
    assert np.all((sig >= 0.1) & (sig <= 10))
    # the row maximum sits close to -ln sigma (z near 0)
    mx = w.x.max(axis=1).astype(np.float64)
    assert np.all(mx <= -np.log(sig) + 1e-6)
    assert np.all(mx >= -np.log(sig) - 0.5 / sig ** 2 * 0.01)


def test_config5_dirichlet_and_dead_rows():
    w = workloads.make(5, rows=1 << 16, aux=True)
    assert np.allclose(w.aux["p"].sum(axis=1), 1.0)
    frac = 1 - w.aux["keep"].mean()
    assert 0.095 < frac < 0.105
    neg = workloads.allneg_rows()
    assert len(neg) == (1 << 24) // 1024 and len(np.unique(neg)) == len(neg)
    local = neg[neg < (1 << 16)]
    assert np.all(np.isneginf(w.x[local]))
    assert np.array_equal(local, w.aux["allneg"])


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_prefix_equals_rows_of_larger_draw(cfg):
    n = workloads.SPECS[cfg].chunk_rows
    a = workloads.make(cfg, rows=n + 3)
    b = workloads.make(cfg, rows=n - 1, threads=1)
    assert np.array_equal(a.x[: n - 1].view(np.uint8), b.x.view(np.uint8))
