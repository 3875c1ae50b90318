"""Pins of the oracle's offline calibration (Spanish summary 2.2 A; Russian page
paragraph 2): covariances against brute-force loops, the causal score matrix,
eigenbasis properties, the lemma-based consequence of Theorem 1 (Russian page
paragraph 5) and the clip quantile."""
import math

import numpy as np

import oracle as O
import synth

SIG = 1 / math.sqrt(128)


def test_query_covariance_brute_force():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 5, 128))
    C = np.zeros((128, 128))
    n = 0
    for g in range(2):
        for i in range(5):
            for a in range(128):
                for b in range(128):
                    C[a, b] += q[g, i, a] * q[g, i, b]
            n += 1
    assert np.abs(O.query_covariance(q) - C / n).max() < 1e-13


def test_score_weighted_covariance_brute_force():
    """Loop form: o_n = sum_{m<=n} softmax_m(sig q_n.k_m) v_m, C_S = mean o o^T."""
    rng = np.random.default_rng(1)
    G, N = 2, 6
    q = rng.standard_normal((G, N, 128))
    k = rng.standard_normal((N, 128))
    v = rng.standard_normal((N, 128))
    C = np.zeros((128, 128))
    for g in range(G):
        for n in range(N):
            lg = [SIG * float(q[g, n] @ k[m]) for m in range(n + 1)]
            mx = max(lg)
            w = [math.exp(x - mx) for x in lg]
            o = sum(w[m] * v[m] for m in range(n + 1)) / sum(w)
            C += np.outer(o, o)
    assert np.abs(O.score_weighted_covariance(q, k, v, SIG) - C / (G * N)).max() < 1e-12


def test_causal_first_row_is_first_value():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 128))
    v = rng.standard_normal((1, 128))
    assert np.abs(O.score_weighted_covariance(q, k, v, SIG) - np.outer(v[0], v[0])).max() < 1e-13


def test_eigenbasis_properties():
    rng = np.random.default_rng(3)
    A = rng.standard_normal((300, 128))
    C = A.T @ A / 300
    U, lam = O.eigenbasis(C)
    assert np.abs(C @ U - U * lam).max() < 1e-10
    assert np.abs(U.T @ U - np.eye(128)).max() < 1e-12
    assert (np.diff(lam) <= 0).all()
    idx = np.argmax(np.abs(U), axis=0)
    assert (U[idx, np.arange(128)] > 0).all()


def test_theorem_consequence_equal_diagonal():
    """With U_Q the eigenbasis of C_Q, R_K = U_Q H P makes every diagonal entry
    of R_K^T C_Q R_K equal tr(C_Q)/d (U_Q diagonalises, then the lemma)."""
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 512, 128)) * np.linspace(0.2, 3, 128)
    C = O.query_covariance(q)
    U, _ = O.eigenbasis(C)
    R = U @ O.hadamard() @ O.bitrev_permutation()
    d = np.diag(R.T @ C @ R)
    assert np.abs(d - np.trace(C) / 128).max() < 1e-12 * np.trace(C)
    # the unrotated channels are far from equal
    assert np.diag(C).max() / np.diag(C).min() > 50


def test_calibrate_layer_clip_quantile_and_shapes():
    rng = np.random.default_rng(0)
    law = synth.outlier_law(rng, 2)
    qc, kc, vc = synth.calibration_samples(rng, law, 2, 512)
    cal = O.calibrate_layer(qc, kc, vc, SIG)
    assert cal["u_k"].shape == (2, 128, 128) and cal["u_k"].dtype == np.uint16
    n = 2 * 512 * 128
    for name, x, U in (("clip_k", kc, cal["u_k"]), ("clip_v", vc, cal["u_v"])):
        rot = np.concatenate([np.abs(x[h] @ O.rotation(U[h])).ravel() for h in range(2)])
        above = int((rot > cal[name]).sum())
        assert abs(above - 0.001 * (n - 1)) <= 2, (name, above)
    # bf16 U stays within bf16 rounding of the fp64 eigenbasis
    # (nearest rounding to 8 significant bits: error <= 2^-8 |x| per entry)
    assert (np.abs(O.bf16_to_f64(cal["u_k"]) - cal["U_Q"]) <= 2 ** -8 * np.abs(cal["U_Q"])).all()
