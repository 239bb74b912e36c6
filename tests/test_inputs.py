"""The seeded input recipe: the fast bfloat16 bit-pattern path gives exactly the values of the float32 path."""
import numpy as np

from linear_rnn_layers_amd import inputs


def _widen(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def test_bf16_bits_match_rounding():
    x = inputs.gaussian((4096,), 77, 3.0)
    # ties and near-ties: values whose lower 16 bits are exactly 0x8000 or one off
    u = x.view(np.uint32).copy()
    u[:64] = (u[:64] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u[64:128] = (u[64:128] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    u[128:192] = (u[128:192] & np.uint32(0xFFFF0000)) | np.uint32(0x8001)
    x = u.view(np.float32)
    assert np.array_equal(_widen(inputs.bf16_bits(x)), inputs.round_to_bf16(x))


def test_gaussian_bits_equal_gaussian_bf16():
    for shape, seed, sigma in (((3, 5, 64), 9, 1.0), ((2, 2, 17, 32), 123, 0.5)):
        a = inputs.gaussian(shape, seed, sigma, inputs.BF16)
        b = _widen(inputs.gaussian_bf16_bits(shape, seed, sigma))
        assert np.array_equal(a, b)


def test_decode_step_bits_equal_the_recipe():
    w = inputs.DECODE
    small = inputs.Workload("d", 3, 2, 4, w.D, w.M, inputs.BF16, 1.0, w.seeds, steps=4)
    for step in (0, 1, 4095):
        ref = small.decode_step_inputs(step)
        got = small.decode_step_bits(step)
        for r, g in zip(ref, got):
            assert np.array_equal(r, _widen(g))
