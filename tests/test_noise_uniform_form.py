"""The kernels form the Gumbel noise's uniform u = (2 (w >> 9) + 1) 2^-24 as
x - (1 - 2^-24), x the float with exponent 0 and mantissa w >> 9 (one
v_alignbit_b32 and one subtraction).  Checked here for all 2^23 values of
w >> 9 in IEEE binary32 arithmetic (round to nearest, as v_add_f32): the
subtraction is exact, so u is bit-identical to the definition the oracle
uses (noise definition of the pages' sampling step, Gumbel-max form)."""
import numpy as np


def test_uniform_via_mantissa_is_exact_for_every_word():
    k = np.arange(1 << 23, dtype=np.uint32)                    # w >> 9
    x = (np.uint32(0x3F800000) | k).view(np.float32)          # 1 + k 2^-23
    one_minus = np.array([0x3F7FFFFF], dtype=np.uint32).view(np.float32)[0]  # 1 - 2^-24
    assert float(one_minus) == 1.0 - 2.0 ** -24
    u_fast = x - one_minus                                     # float32 - float32, rounded to nearest
    u_def = ((2 * k.astype(np.uint64) + 1).astype(np.float64) * 2.0 ** -24).astype(np.float32)
    assert u_def.dtype == np.float32 and u_fast.dtype == np.float32
    assert np.array_equal(u_fast.view(np.uint32), u_def.view(np.uint32))
    # the definition itself is exact in float32 (at most 24 significant bits)
    assert np.array_equal(u_def.astype(np.float64), (2 * k.astype(np.float64) + 1) * 2.0 ** -24)
    assert u_fast.min() == np.float32(2.0 ** -24) and u_fast.max() == np.float32(1.0 - 2.0 ** -24)
