"""Pins of the oracle's Hadamard transform: scipy's Sylvester matrix,
orthogonality, inverse, norm preservation, closed forms, sign placement."""
import numpy as np
import pytest
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


def _spike_tensor(rows, cols, axis, rng):
    """One spike per 16-chunk along `axis`, magnitude 2^-k (k = 0..3) with a
    random sign at a random position; returns x and the per-chunk (c, position)."""
    n_chunks = (rows, cols // 16) if axis == "row" else (rows // 16, cols)
    k = rng.integers(0, 4, n_chunks)
    k[0, 0] = 0  # the tensor maximum is 1
    c = np.where(rng.random(n_chunks) < 0.5, -1.0, 1.0) * np.exp2(-k)
    pos = rng.integers(0, 16, n_chunks)
    x = np.zeros((rows, cols))
    for i in range(n_chunks[0]):
        for j in range(n_chunks[1]):
            if axis == "row":
                x[i, 16 * j + pos[i, j]] = c[i, j]
            else:
                x[16 * i + pos[i, j], j] = c[i, j]
    return x, c, pos, k


@pytest.mark.parametrize("axis", ["row", "col"])
def test_rht_nvfp4_of_spikes_closed_form(axis):
    # a spike c at position p of a chunk transforms to (c/4) s_p H[:, p]: sixteen
    # values of magnitude |c|/4, so the transformed amax is 1/4, every 16-block
    # (one chunk) has scale 448 * |c| (E4M3 exact for |c| = 2^-k) and every code is
    # +-6 with the sign of c s_p H[i][p]
    rng = np.random.default_rng(11)
    mask = 0b1010011000110101
    x, c, pos, k = _spike_tensor(32, 64, axis, rng)
    assert rht.rht_amax(x, mask, axis) == 0.25
    codes, sb, st = (rht.rht_nvfp4_rowwise if axis == "row" else rht.rht_nvfp4_colwise)(x, mask)
    assert st == np.float32(0.25 / 2688)
    h = scipy.linalg.hadamard(16)
    s = rht.signs_from_mask(mask)
    cm = c if axis == "row" else c.T
    pm = pos if axis == "row" else pos.T
    km = k if axis == "row" else k.T
    expect_sb = {0: 0x7E, 1: 0x76, 2: 0x6E, 3: 0x66}  # E4M3 of 448, 224, 112, 56
    assert np.array_equal(sb, np.vectorize(expect_sb.get)(km))
    got = mx.unpack_nibbles(codes)
    R2, C2 = got.shape
    for i in range(R2):
        for j in range(C2 // 16):
            sign = np.sign(cm[i, j] * s[pm[i, j]] * h[:, pm[i, j]])
            expect = np.where(sign < 0, 0x8 | 7, 7)
            assert np.array_equal(got[i, 16 * j:16 * j + 16], expect), (i, j)


def test_rht_amax_orders_and_axes():
    # the transform is orthonormal per chunk: the amax of y lies between the chunk
    # norm / 4 and the chunk norm, for either axis
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 96))
    for axis in ("row", "col"):
        xa = x if axis == "row" else x.T
        n = np.linalg.norm(xa.reshape(xa.shape[0], -1, 16), axis=-1)
        a = rht.rht_amax(x, 0x1234, axis)
        assert n.max() / 4 <= a <= n.max() + 1e-12
