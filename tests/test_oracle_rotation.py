"""Pins of the oracle's rotation factors against facts the pages and the
mathematics fix: the Walsh-Hadamard matrix (closed form, library routine, fast
transform, the lemma of the Russian page, paragraph 5), the bit-reversal
involution, orthogonality of R (Russian page paragraph 2) and the factor order /
orientation R = U H P (Italian page "I tre fattori della rotazione"; Spanish
summary 2.2 A.3)."""
import numpy as np
import pytest
import scipy.linalg

import oracle as O


def popcount(x):
    return bin(int(x)).count("1")


def test_hadamard_closed_form():
    H = O.hadamard(128)
    ref = np.array([[(-1) ** popcount(i & j) for j in range(128)] for i in range(128)]) / np.sqrt(128)
    assert np.array_equal(H, ref)


def test_hadamard_matches_library_sylvester():
    assert np.allclose(O.hadamard(128), scipy.linalg.hadamard(128) / np.sqrt(128), atol=0, rtol=0)


def test_hadamard_orthonormal_symmetric():
    H = O.hadamard(128)
    assert np.array_equal(H, H.T)
    assert np.abs(H @ H.T - np.eye(128)).max() < 1e-14


def fwht(x):
    """In-place radix-2 butterflies (a different algorithm from the matrix)."""
    x = np.array(x, np.float64)
    h = 1
    while h < x.shape[-1]:
        for i in range(0, x.shape[-1], 2 * h):
            a = x[..., i:i + h].copy()
            b = x[..., i + h:i + 2 * h].copy()
            x[..., i:i + h] = a + b
            x[..., i + h:i + 2 * h] = a - b
        h *= 2
    return x / np.sqrt(x.shape[-1])


def test_fast_transform_equals_matrix():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 128))
    assert np.abs(fwht(x) - x @ O.hadamard(128)).max() < 1e-13


def test_lemma_diagonal_equalisation():
    """diag(H Lambda H^T) = tr(Lambda)/d for any diagonal Lambda (Russian page,
    paragraph 5).  Only the orthonormal H satisfies it."""
    rng = np.random.default_rng(2)
    H = O.hadamard(128)
    for _ in range(5):
        lam = rng.exponential(size=128) * 10 ** rng.uniform(-2, 2, size=128)
        M = H @ np.diag(lam) @ H.T
        assert np.abs(np.diag(M) - lam.sum() / 128).max() < 1e-12 * lam.sum()
    # unnormalised Sylvester gives tr(Lambda), not tr(Lambda)/d
    S = H * np.sqrt(128)
    M = S @ np.diag(lam) @ S.T
    assert not np.allclose(np.diag(M), lam.sum() / 128)


def test_bitrev_values_and_involution():
    br = O.bitrev7(np.arange(128))
    assert br[0] == 0 and br[1] == 64 and br[2] == 32 and br[3] == 96 and br[5] == 80
    assert br[127] == 127 and br[64] == 1
    assert np.array_equal(br[br], np.arange(128))
    assert sorted(br) == list(range(128))


def test_bitrev_permutation_matrix():
    P = O.bitrev_permutation()
    assert np.array_equal(P, P.T)
    assert np.array_equal(P @ P, np.eye(128))
    z = np.arange(128, dtype=np.float64)
    w = z @ P
    # (z P)_j = z_{br(j)}; group 0 of w (j < 64) holds exactly the even z channels
    assert np.array_equal(w, z[O.bitrev7(np.arange(128))])
    assert sorted(w[:64]) == list(range(0, 128, 2))
    assert sorted(w[64:]) == list(range(1, 128, 2))


def test_rotation_orthogonal_fp64_and_bf16():
    rng = np.random.default_rng(3)
    U, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    R64 = U @ O.hadamard() @ O.bitrev_permutation()
    assert np.abs(R64.T @ R64 - np.eye(128)).max() < 1e-12
    R = O.rotation(O.f64_to_bf16(U))
    assert np.abs(R.T @ R - np.eye(128)).max() < 8e-3


def test_rotation_orientation_pin():
    """With C = U Lambda U^T and U orthogonal, non-diagonalising-trivially and
    exactly representable in bf16 (a permuted block diagonal of 4x4 Hadamard
    blocks, entries +-1/2), R = U H P gives diag(R^T C R) = tr(C)/d exactly:
    U diagonalises C, then the lemma applies.  U applied last or transposed
    does not."""
    rng = np.random.default_rng(4)
    H4 = scipy.linalg.hadamard(4) / 2.0
    B = np.kron(np.eye(32), H4)
    perm = rng.permutation(128)
    U = B[perm] * rng.choice([-1.0, 1.0], 128)[None, :]
    assert np.abs(U @ U.T - np.eye(128)).max() == 0
    lam = rng.exponential(size=128) * 10
    C = U @ np.diag(lam) @ U.T
    assert np.abs(C - np.diag(np.diag(C))).max() > 1.0      # C is not diagonal
    R = O.rotation(O.f64_to_bf16(U))
    d = np.diag(R.T @ C @ R)
    assert np.abs(d - np.trace(C) / 128).max() < 1e-12 * np.trace(C)
    H, P = O.hadamard(), O.bitrev_permutation()
    for wrong in (H @ U @ P, U.T @ H @ P, H @ P @ U):
        dw = np.diag(wrong.T @ C @ wrong)
        assert np.abs(dw - np.trace(C) / 128).max() > 1e-3 * np.trace(C)


def test_rotate_equals_dense_rotation():
    rng = np.random.default_rng(5)
    U = O.f64_to_bf16(np.linalg.qr(rng.standard_normal((128, 128)))[0])
    x = rng.standard_normal((9, 128))
    assert np.abs(O.rotate(x, U) - x @ O.rotation(U)).max() < 1e-13
