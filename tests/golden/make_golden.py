"""Write tests/golden/edge_cases.txt: small edge-case inputs and the oracle's values.

Run from the repository root: ``python tests/golden/make_golden.py``. It calls
only the float64 oracle (``oracle/``) and numpy; no value here comes from the
HIP library. Each case cites the passage of the paper ("Speeding up
Log-Sum-Exp: Kernel Fusion at the Memory Wall, Integer Arithmetic at the
Compute Wall") or the reading that defines it.

File format, one case per block:
    case <name>
    cite <text>
    dtype f32|bf16
    shape <rows> <cols>
    x <hex element bit patterns, row-major, space separated>
    out <float.hex of each row's float64 LSE>
"""
import math
import sys
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

import oracle  # noqa: E402

OUT = Path(__file__).resolve().parent / "edge_cases.txt"
INF, NAN = np.inf, np.nan


def f32(rows):
    return np.array(rows, dtype=np.float32)


def bf16(rows):
    a = np.array(rows, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)  # values chosen bf16-exact


def cases():
    rng = np.random.default_rng(2024)
    yield ("special_values_f32",
           "Table 3 lists edge-case handling without cells; torch.logsumexp semantics "
           "(the paper's drop-in target, abstract)",
           f32([[-INF, -INF, -INF, -INF], [1.0, NAN, 2.0, 0.0], [INF, 1.0, -INF, 0.0],
                [INF, NAN, 0.0, 0.0], [-INF, 0.0, -INF, 0.0], [-INF, NAN, -INF, -INF]]))
    yield ("special_values_bf16", "as special_values_f32, bf16 storage",
           bf16([[-INF, -INF, -INF], [1.0, NAN, 2.0], [INF, 1.0, -INF], [-INF, 0.5, -INF]]))
    yield ("constant_rows",
           "closed form c + ln N of the LSE definition (title, abstract)",
           f32([[3.25] * 33, [-40.0] * 33, [0.0] * 33]))
    yield ("pairs", "the pairwise operator, f(z) = log2(1 + 2^z) (§A.1)",
           f32([[0.0, 0.0], [800.0, 0.0], [-1000.0, 1000.0], [3.5, -2.25], [-60.0, -61.0]]))
    yield ("huge_magnitudes",
           "values near the fp32 range end: LSE = max + ln(count), no overflow",
           f32([[3.0e38, 3.0e38, -1.0], [-3.0e38, -3.0e38, -3.0e38], [1.0e38, -1.0e38, 0.0],
                [2.0e38, 1.0, 2.0e38]]))
    yield ("below_underflow",
           "terms more than 87.3 below the row max underflow in fp32 (Table 5)",
           f32([[0.0, -87.0, -88.0, -100.0, -104.0, -150.0], [-5.0, -92.3, -193.0, -5.0, -6.0, -7.0]]))
    yield ("subnormals", "fp32 subnormal inputs are used unflushed by the oracle",
           f32([[1e-45, -INF, 1e-44], [-1e-40, 1e-40, 0.0]]))
    for cols in (1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 33, 63, 65):
        yield (f"ragged_f32_{cols}", "row-wise reduction over N of a (B, N) tensor (§2.1, §3.1)",
               rng.normal(0, 6, size=(5, cols)).astype(np.float32))
    for cols in (1, 3, 7, 8, 9, 15, 16, 17, 33):
        v = rng.normal(0, 6, size=(4, cols)).astype(np.float32)
        yield (f"ragged_bf16_{cols}", "as ragged_f32, bf16 storage (bits rounded toward zero)",
               (v.view(np.uint32) >> 16).astype(np.uint16))


def main():
    orc = oracle.default()
    lines = []
    for name, cite, x in cases():
        dtype = "bf16" if x.dtype == np.uint16 else "f32"
        out = orc.lse(x, dtype)
        width = 4 if dtype == "bf16" else 8
        bits = x.view(np.uint16 if dtype == "bf16" else np.uint32).ravel()
        lines += [f"case {name}", f"cite {cite}", f"dtype {dtype}",
                  f"shape {x.shape[0]} {x.shape[1]}",
                  "x " + " ".join(f"{int(b):0{width}x}" for b in bits),
                  "out " + " ".join(float(v).hex() if not math.isnan(v) else "nan" for v in out),
                  ""]
    OUT.write_text("\n".join(lines))
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
