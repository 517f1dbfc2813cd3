"""Pins of the oracle's randomized Hadamard rotation (ai-paper-analysis page, section 3.1:
H H^T = I, so Q K^T is unchanged when Q is rotated too, and rotation keeps vector length).
"""
import numpy as np
import pytest
import scipy.linalg

from oracle import kvarn_ref as R
from kv_cache_bit_amd import synth


def fwht_butterfly(x):
    """Independent fast Walsh-Hadamard transform (iterative butterflies, no matrix)."""
    a = np.array(x, dtype=np.float64)
    n = a.shape[-1]
    h = 1
    while h < n:
        a = a.reshape(a.shape[:-1] + (n // (2 * h), 2, h))
        lo = a[..., 0, :].copy()
        hi = a[..., 1, :].copy()
        a[..., 0, :] = lo + hi
        a[..., 1, :] = lo - hi
        a = a.reshape(a.shape[:-3] + (n,))
        h *= 2
    return a


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_sylvester_is_hadamard_integer(d):
    h = R.hadamard_sylvester(d)
    assert np.array_equal(h @ h.T, d * np.eye(d, dtype=np.int64))
    assert np.array_equal(h, scipy.linalg.hadamard(d))          # library Sylvester construction


def test_sylvester_recursion():
    h = np.array([[1]])
    for _ in range(7):
        h = np.block([[h, h], [h, -h]])
    assert np.array_equal(R.hadamard_sylvester(128), h)


@pytest.mark.parametrize("seed", [0, 1, 7])
def test_rotation_orthonormal(seed):
    s = synth.sign_vector(seed, 128)
    m = R.rotation_matrix(s)
    assert np.abs(m @ m.T - np.eye(128)).max() < 1e-15 * 128


def test_rotation_equals_butterfly_transform():
    rng = np.random.default_rng(3)
    s = synth.sign_vector(5, 128).astype(np.float64)
    x = rng.standard_normal((17, 128))
    assert np.allclose(R.rotate(x, s), fwht_butterfly(x * s) / np.sqrt(128), rtol=0, atol=1e-13)


def test_rotation_unit_vectors_and_ones():
    d = 128
    ones = np.ones(d)
    # all-ones input with sigma = 1 -> sqrt(D) e_0
    w = R.rotate(ones, ones)
    e0 = np.zeros(d)
    e0[0] = np.sqrt(d)
    assert np.abs(w - e0).max() < 1e-13
    # e_k -> row k of H_D
    s = synth.sign_vector(0, d).astype(np.float64)
    eye = np.eye(d)
    assert np.abs(R.rotate(eye, s) - R.rotation_matrix(s)).max() == 0


def test_rotation_preserves_norm_and_scores():
    rng = np.random.default_rng(4)
    s = synth.sign_vector(11, 128)
    q = rng.standard_normal((3, 128))
    k = rng.standard_normal((50, 128)) * 10
    assert np.allclose(np.linalg.norm(R.rotate(k, s), axis=-1), np.linalg.norm(k, axis=-1), rtol=1e-14)
    assert np.abs(R.rotate(q, s) @ R.rotate(k, s).T - q @ k.T).max() < 1e-12 * np.abs(q @ k.T).max()
    assert np.abs(R.unrotate(R.rotate(k, s), s) - k).max() < 1e-12
