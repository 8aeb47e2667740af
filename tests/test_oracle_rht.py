"""Pins of the oracle's Hadamard transform: scipy's Sylvester matrix,
orthogonality, inverse, norm preservation, closed forms, sign placement."""
import numpy as np
import scipy.linalg

from oracle import mx, rht


def test_h16_is_scipy_sylvester_and_orthogonal():
    h = rht.sylvester_h16()
    np.testing.assert_array_equal(h, scipy.linalg.hadamard(16).astype(np.float64))
    np.testing.assert_array_equal(h @ h.T, 16 * np.eye(16))


def test_constant_chunk_maps_to_first_coefficient():
    x = np.full((1, 32), 3.0)
    y = rht.rht_rowwise(x, 0)
    expect = np.zeros(32)
    expect[0] = expect[16] = 12.0  # (1/4) * 16 * 3
    np.testing.assert_array_equal(y[0], expect)


def test_sign_bit_i_flips_input_i():
    h = scipy.linalg.hadamard(16).astype(np.float64)
    for i in range(16):
        x = np.zeros((1, 16))
        x[0, i] = 1.0
        np.testing.assert_array_equal(rht.rht_rowwise(x, 0)[0], 0.25 * h[:, i])
        np.testing.assert_array_equal(rht.rht_rowwise(x, 1 << i)[0], -0.25 * h[:, i])
        np.testing.assert_array_equal(rht.rht_rowwise(x, 0xFFFF ^ (1 << i))[0], 0.25 * h[:, i])


def test_inverse_and_norm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((8, 64))
    for mask in (0, 0xA5C3, 0xFFFF):
        y = rht.rht_rowwise(x, mask)
        # inverse: x = s * (1/4) H y (H symmetric, s^2 = 1)
        s = rht.signs_from_mask(mask)
        back = (y.reshape(8, 4, 16) @ scipy.linalg.hadamard(16).T * 0.25) * s
        np.testing.assert_allclose(back.reshape(8, 64), x, rtol=0, atol=1e-13)
        np.testing.assert_allclose(np.linalg.norm(y.reshape(8, 4, 16), axis=-1),
                                   np.linalg.norm(x.reshape(8, 4, 16), axis=-1), rtol=1e-14)


def test_colwise_is_rowwise_of_transpose():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 48))
    p1, s1 = rht.rht_mxfp4_colwise(x, 0x1234)
    p2, s2 = mx.mxfp4_quantize_rowwise(rht.rht_rowwise(x.T.copy(), 0x1234))
    np.testing.assert_array_equal(p1, p2)
    np.testing.assert_array_equal(s1, s2)


def test_spreads_an_outlier():
    x = np.zeros((1, 32))
    x[0, 3] = 100.0
    x[0, 1] = 1.0
    y = rht.rht_rowwise(x, rht.sign_mask_from_seed(4))
    assert np.abs(y[0, :16]).max() < 30  # energy of the spike shared by 16 outputs


def test_sign_mask_from_seed_is_16_bits_and_seed_dependent():
    masks = {rht.sign_mask_from_seed(s) for s in range(64)}
    assert all(0 <= m < 65536 for m in masks)
    assert len(masks) > 60
