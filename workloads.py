"""Seeded synthetic inputs for the row-wise log-sum-exp.

This module draws the five input matrices that the tests and the benchmark
use. It does no log-sum-exp arithmetic of its own: it only draws random
numbers, shapes them into the stated distributions and rounds them to the
storage type. Both the float64 oracle and the GPU path read what it returns.

The five workloads stand in for the applications that the source paper
("Speeding up Log-Sum-Exp: Kernel Fusion at the Memory Wall, Integer
Arithmetic at the Compute Wall", §2 and §5) benchmarks on data that is not
available here:

* 1 - fp32 [64, 32000], x ~ N(0, 3^2): short LLM-vocabulary rows (§5.1).
* 2 - bf16 [512, 128256], logits ~ N(0, 2^2) with 8 spike columns per row
  set to 15, plus a per-row offset ~ U(-20, 20): the (B, N) shape that the
  paper profiles in Figure 1 (§2.1).
* 3 - bf16 [4096, 262144], x ~ N(0, 4^2) with 1 % of entries -inf: the
  largest RLHF vocabulary (§5.1).
* 4 - fp32 [65536, 4096], particle-filter log-weights
  x_ij = -z_ij^2 / (2 sigma_i^2) - ln sigma_i, z ~ N(0, 1),
  sigma_i ~ U(0.1, 10) (§5.3).
* 5 - fp32 [16777216, 16], log of a Dirichlet(0.5) sample per row, 10 % of
  entries -inf and 16384 rows entirely -inf: probabilistic-circuit sum
  nodes (§5.2).

Determinism: rows are drawn in fixed chunks. Chunk i of every workload uses
``numpy.random.default_rng(SeedSequence(0, spawn_key=(i,)))``, which is the
i-th child of seed 0, so any prefix of rows can be regenerated alone and is
bit-identical to the same rows of the full matrix. bf16 values are stored as
their uint16 bit patterns, rounded from fp32 to nearest-even; ``make(...,
storage="f16")`` stores the same fp32 draws as IEEE half bit patterns instead
(``storage="f32"`` keeps them unrounded).
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

SEED = 0

# Spawn key of the generator that picks config 5's all -inf rows; chunk keys
# stay far below it.
_ALLNEG_KEY = 0xFFFF_FFFF


@dataclass(frozen=True)
class Spec:
    cfg: int
    name: str
    dtype: str  # "f32", "bf16" or "f16": the storage type of x
    rows: int
    cols: int
    chunk_rows: int
    recipe: str


SPECS = {
    1: Spec(1, "fp32_64x32000_normal3", "f32", 64, 32000, 64,
            "x ~ N(0, 3^2) drawn in fp32"),
    2: Spec(2, "bf16_512x128256_spiky_vocab", "bf16", 512, 128256, 32,
            "z ~ N(0, 2^2) in fp32; 8 distinct columns per row set to 15; "
            "x = z + o_i with o_i ~ U(-20, 20); RNE to bf16"),
    3: Spec(3, "bf16_4096x262144_normal4_neginf", "bf16", 4096, 262144, 16,
            "x ~ N(0, 4^2) in fp32; each entry -inf with probability 0.01; "
            "RNE to bf16"),
    4: Spec(4, "fp32_65536x4096_particle_logw", "f32", 65536, 4096, 1024,
            "sigma_i ~ U(0.1, 10), z ~ N(0, 1), "
            "x = -z^2/(2 sigma_i^2) - ln sigma_i in float64, then fp32"),
    5: Spec(5, "fp32_16777216x16_dirichlet_logp", "f32", 1 << 24, 16, 1 << 16,
            "p ~ Dirichlet(0.5 * 1_16) in float64, x = ln p rounded to fp32; "
            "each entry -inf with probability 0.1; 16384 rows (1/1024, drawn "
            "without replacement) entirely -inf"),
}


@dataclass
class Workload:
    spec: Spec
    x: np.ndarray          # [rows, cols] float32, or uint16 bf16 / fp16 bit patterns
    rows: int
    aux: dict = field(default_factory=dict)

    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def cols(self) -> int:
        return self.spec.cols

    @property
    def nbytes(self) -> int:
        return self.x.nbytes


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, nearest-even, returning uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE half, nearest-even (numpy's cast), returning
    uint16 bits; beyond the half range they become +-inf."""
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(SEED, spawn_key=(key,)))


# ---- per-chunk generators: each returns (x_chunk, aux_chunk) -----------------

def _chunk1(rng, n, cols, want_aux):
    x = rng.standard_normal((n, cols), dtype=np.float32)
    x *= np.float32(3.0)
    return x, {}


def _chunk2(rng, n, cols, want_aux):
    z = rng.standard_normal((n, cols), dtype=np.float32)
    z *= np.float32(2.0)
    spikes = np.empty((n, 8), dtype=np.int64)
    for i in range(n):
        spikes[i] = rng.choice(cols, size=8, replace=False)
    z[np.arange(n)[:, None], spikes] = np.float32(15.0)
    off = rng.uniform(-20.0, 20.0, size=n).astype(np.float32)
    z += off[:, None]
    aux = {"offset": off, "spikes": spikes} if want_aux else {}
    return z, aux


def _chunk3(rng, n, cols, want_aux):
    x = rng.standard_normal((n, cols), dtype=np.float32)
    x *= np.float32(4.0)
    x[rng.random((n, cols), dtype=np.float32) < np.float32(0.01)] = -np.inf
    return x, {}


def _chunk4(rng, n, cols, want_aux):
    sigma = rng.uniform(0.1, 10.0, size=n)
    z = rng.standard_normal((n, cols))
    x = (-0.5 * z * z / (sigma * sigma)[:, None] - np.log(sigma)[:, None]).astype(np.float32)
    return x, ({"sigma": sigma} if want_aux else {})


def _chunk5(rng, n, cols, want_aux):
    p = rng.dirichlet(np.full(cols, 0.5), size=n)
    keep = rng.random((n, cols)) >= 0.1
    x = np.log(p).astype(np.float32)
    x[~keep] = -np.inf
    return x, ({"p": p, "keep": keep} if want_aux else {})


_CHUNK = {1: _chunk1, 2: _chunk2, 3: _chunk3, 4: _chunk4, 5: _chunk5}


def allneg_rows(total_rows: int = 1 << 24) -> np.ndarray:
    """Sorted indices of config 5's entirely -inf rows (1/1024 of all rows)."""
    sel = _rng(_ALLNEG_KEY).choice(total_rows, size=total_rows // 1024, replace=False)
    return np.sort(sel)


_ROUND = {"bf16": f32_to_bf16_bits, "f16": f32_to_f16_bits}


def make(cfg: int, rows: int | None = None, aux: bool = False,
         threads: int | None = None, storage: str | None = None) -> Workload:
    """Return workload ``cfg`` or the prefix of its first ``rows`` rows.

    A prefix holds exactly the same values as the same rows of the full
    matrix. ``aux=True`` also returns the generator's own draws (offsets,
    spike columns, sigma, the Dirichlet p and keep mask, the all -inf rows)
    for the tests that check the workloads against their definitions.
    ``storage`` ("f32", "bf16" or "f16") overrides the stored element type:
    the same seeded fp32 values, kept or rounded to nearest-even in the other
    16-bit format (the paper's reduced-bit comparison, §4.3).
    """
    spec = SPECS[cfg]
    if storage is not None and storage != spec.dtype:
        if storage not in ("f32", "bf16", "f16"):
            raise ValueError(f"unknown storage {storage!r}")
        spec = replace(spec, dtype=storage, name=spec.name.replace(spec.dtype, storage, 1)
                       .replace("fp32", storage, 1),
                       recipe=spec.recipe.replace("RNE to bf16", f"stored as {storage}")
                       if "RNE to bf16" in spec.recipe else spec.recipe + f"; stored as {storage}")
    n = spec.rows if rows is None else int(rows)
    if not 0 <= n <= spec.rows:
        raise ValueError(f"rows must be in [0, {spec.rows}]")
    store = np.float32 if spec.dtype == "f32" else np.uint16
    rnd = _ROUND.get(spec.dtype)
    x = np.empty((n, spec.cols), dtype=store)
    nchunks = -(-n // spec.chunk_rows)
    auxes: list[dict] = [dict() for _ in range(nchunks)]

    def one(i: int) -> None:
        r0 = i * spec.chunk_rows
        full = min(spec.chunk_rows, spec.rows - r0)
        xc, ac = _CHUNK[cfg](_rng(i), full, spec.cols, aux)
        take = min(full, n - r0)
        x[r0:r0 + take] = rnd(xc[:take]) if rnd is not None else xc[:take]
        auxes[i] = {k: v[:take] for k, v in ac.items()}

    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    if nchunks <= 1 or threads <= 1:
        for i in range(nchunks):
            one(i)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(nchunks)))

    out_aux: dict = {}
    if aux and nchunks:
        for k in auxes[0]:
            out_aux[k] = np.concatenate([a[k] for a in auxes])
    if cfg == 5:
        neg = allneg_rows(spec.rows)
        neg = neg[neg < n]
        x[neg] = -np.inf if rnd is None else rnd(np.array([-np.inf], dtype=np.float32))[0]
        if aux:
            out_aux["allneg"] = neg
    return Workload(spec=spec, x=x, rows=n, aux=out_aux)


_TARGET_KEY = 1 << 40  # spawn key of the target-column stream, apart from the chunk keys


def targets(cfg: int, rows: int | None = None) -> np.ndarray:
    """Seeded target columns for the token log-probability workloads: one
    uniform draw from [0, cols) per row (the sampled token of each position),
    int64. A prefix of rows matches the same rows of the full draw."""
    spec = SPECS[cfg]
    n = spec.rows if rows is None else int(rows)
    if not 0 <= n <= spec.rows:
        raise ValueError(f"rows must be in [0, {spec.rows}]")
    t = _rng(_TARGET_KEY).integers(0, spec.cols, size=spec.rows, dtype=np.int64)
    return t[:n].copy()


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8).data).hexdigest()
