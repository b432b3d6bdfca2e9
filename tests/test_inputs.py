"""The seeded input generator: bf16 rounding, determinism and workload recipe (CPU)."""
import numpy as np

from synth import inputs


def test_bf16_round_nearest_even():
    f = np.array([1.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, 1.0 + 2.0**-9, -2.5, 0.0,
                  1.0 + 2.0**-8 + 2.0**-20, 3.0e38], dtype=np.float32)
    got = inputs.f32_to_bf16_bits(f)
    # 1+2^-8 is a tie between 0x3F80 and 0x3F81 -> even 0x3F80; 1+3*2^-8 ties -> 0x3F82;
    # just above a tie rounds up; 3e38 rounds to 0x7F62 (largest finite-ish region)
    exp = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F80, 0xC020, 0x0000, 0x3F81, 0x7F62],
                   dtype=np.uint16)
    np.testing.assert_array_equal(got, exp)


def test_deterministic_and_shapes():
    a = inputs.config_case(1)
    b = inputs.config_case(1)
    np.testing.assert_array_equal(a.X, b.X)
    np.testing.assert_array_equal(a.W, b.W)
    np.testing.assert_array_equal(a.targets, b.targets)
    assert a.X.shape == (64, 128) and a.W.shape == (1000, 128)
    assert (a.targets == -100).sum() == 3
    assert a.grad_logprob is not None and np.all(a.grad_logprob == np.float32(1 / 64))
    assert a.grad_entropy is None


def test_chunked_draw_equals_single_draw():
    rng1 = inputs._rng(77, 0)
    one = inputs.f32_to_bf16_bits(rng1.standard_normal(3000 * 50, dtype=np.float32)).reshape(3000, 50)
    two = inputs._normal_bf16(inputs._rng(77, 0), 3000, 50, 1.0, chunk_elems=777)
    np.testing.assert_array_equal(one, two)


def test_big_rows_recipe():
    c = inputs.make_case("b", 5, 200, 16, 300, ignore_frac=0.1, big_rows_frac=0.1,
                         big_factor=64.0, grad_mode="normal")
    plain = inputs.make_case("p", 5, 200, 16, 300, ignore_frac=0.1, grad_mode="normal")
    xf = inputs.decode_bf16_to_f32(c.X)
    pf = inputs.decode_bf16_to_f32(plain.X)
    big = np.where(np.any(xf != pf, axis=1))[0]
    assert len(big) == 20
    np.testing.assert_array_equal(xf[big], pf[big] * 64)
    assert (c.targets == -100).sum() == 20
    assert c.grad_entropy is not None and c.grad_entropy.dtype == np.float32
