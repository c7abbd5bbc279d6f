"""Writes tests/golden/rmsnorm_bf16_order.json.

The M01 drill page states that in bf16 the RMSNorm must cast the normalised
value back to bf16 *before* the weight multiply, and prints one outcome of each
order (correct 1.9140625, multiply-in-fp32-first 1.90625) without printing the
inputs.  This script searches seeded random bf16 rows (eps = 0) for an
instance on which the two orders give exactly those two printed numbers, using
the oracle's own primitives for the correct order and the same primitives with
the cast moved for the other order.  The stored instance then pins the order
rule: the oracle must give 1.9140625 on it.
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))
from oracle import mrope_oracle as O  # noqa: E402

GOOD, BAD = 1.9140625, 1.90625


def main():
    rng = np.random.default_rng(0)
    for _ in range(1_000_000):
        x_bits = O.f32_to_bf16_bits(rng.standard_normal(2).astype(np.float32))
        w_bits = O.f32_to_bf16_bits((1.9 + 0.1 * rng.standard_normal(2)).astype(np.float32))
        x, w = O.bf16_bits_to_f64(x_bits), O.bf16_bits_to_f64(w_bits)
        n = O.fl32(x * O.rms_scale(x, 0.0)).astype(np.float64)
        cast_first = O.bf(O.bf(n) * w)
        mul_first = O.bf(O.fl32(n * w))
        for i in range(2):
            if cast_first[i] == GOOD and mul_first[i] == BAD:
                out = {
                    "cite": "M01 drill page, L1 'details': bf16 RMSNorm order example (correct order "
                            "1.9140625, fp32 multiply first 1.90625); inputs not printed on the page, "
                            "found by tests/golden/make_bf16_order_case.py",
                    "x_bf16_bits": [int(v) for v in x_bits],
                    "w_bf16_bits": [int(v) for v in w_bits],
                    "eps": 0.0,
                    "element": i,
                    "correct": GOOD,
                    "fp32_first": BAD,
                }
                path = os.path.join(os.path.dirname(__file__), "rmsnorm_bf16_order.json")
                with open(path, "w") as f:
                    json.dump(out, f, indent=2)
                print(out)
                return
    raise SystemExit("no instance found")


if __name__ == "__main__":
    main()
