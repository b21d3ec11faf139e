"""CPU checks of the build A/B harness (row_wise_log_amd.ab_builds): its
argument parsing, the input rotation, and that it refuses to run without a
GPU. The timing itself needs a GPU and is not run here."""
import argparse

import pytest

from row_wise_log_amd import ab_builds as A


def test_parse_shape():
    assert A.parse_shape("bf16:512:128256") == ("bf16", 512, 128256)
    assert A.parse_shape("f32:1:3") == ("f32", 1, 3)
    for bad in ("bf16:512", "i8:4:4", "f32:0:5", "f16:3:-1"):
        with pytest.raises(argparse.ArgumentTypeError):
            A.parse_shape(bad)


def test_parse_lib():
    assert A.parse_lib("a/b.so") == (A.Path("a/b.so"), 0)
    assert A.parse_lib("a/b.so:64") == (A.Path("a/b.so"), 64)


def test_rotation_exceeds_twice_the_cache():
    for nbytes in (131334144, 1 << 30, 3 * (1 << 20) + 7):
        assert A.rotation(nbytes) * nbytes > 2 * A.CACHE_BYTES
    assert A.rotation(16) == 4096


def test_needs_two_builds_and_a_gpu(tmp_path):
    with pytest.raises(SystemExit):
        A.main(["--lib", str(tmp_path / "a.so")])
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(SystemExit, match="needs a GPU"):
        A.main(["--lib", str(tmp_path / "a.so"), "--lib", str(tmp_path / "b.so")])
