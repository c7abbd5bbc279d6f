"""The full-size parity comparison (tests/_oracle_pool.py) finds what it must:
bf16 ulp distances across zero and signs, binary32 absolute errors and
bit differences, and chunk totals."""
import numpy as np

from tests import _oracle_pool as OP
import workloads as W


def test_bf16_ulps():
    a = W.to_bf16_bits(np.array([1.0, -2.0, 0.0, 3.0, -0.0], dtype=np.float32))
    b = a.copy()
    assert OP.compare(a, b, "bf16") == (5, 0, 0.0)
    b[0] += 1                      # one ulp up
    b[1] += 2                      # -2 -> two ulps further from zero
    b[4] = 0x0000                  # -0 vs +0: equal
    n, off, worst = OP.compare(b, a, "bf16")
    assert (n, off, worst) == (5, 2, 2.0)
    tiny_pos, tiny_neg = np.array([0x0001], np.uint16), np.array([0x8001], np.uint16)
    assert OP.compare(tiny_pos, tiny_neg, "bf16")[2] == 2.0    # straddles zero


def test_f32_abs_and_bits():
    a = np.array([1.0, 2.0, -3.0], dtype=np.float32)
    b = a.copy()
    b[2] = np.nextafter(np.float32(-3.0), np.float32(0.0))
    n, off, worst = OP.compare(b, a, "f32")
    assert n == 3 and off == 1 and 0 < worst < 1e-6
    b[0] = 1.5
    assert OP.compare(b, a, "f32")[2] == 0.5


def test_merge_sums_chunks():
    assert OP.merge([(10, 1, 1.0), (5, 0, 0.0), (7, 3, 2.0)]) == (22, 4, 2.0)
