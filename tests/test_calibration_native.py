"""Parity of the library's host calibration (C++, oscar_calibrate_layer)
with the oracle's (NumPy fp64), on seeded synthetic calibration sets.
Offline calibration: Spanish summary section 2.2 A; Russian page paragraph 2."""
import math

import numpy as np
import pytest

import int2_rotated_kv_write_amd as lib
import oracle as O
import synth

SIG = 1 / math.sqrt(128)


@pytest.mark.parametrize("H,G,N,law", [(1, 4, 2048, "outlier"), (2, 2, 300, "heavy"), (3, 1, 200, "outlier")])
def test_native_calibration_matches_oracle(H, G, N, law):
    # G*N >= 128 keeps the spectra free of exact degeneracy, so the canonical
    # eigenbasis is unique and both implementations must find the same one.
    rng = np.random.default_rng(H * 100 + G)
    kv = synth.outlier_law(rng, H) if law == "outlier" else synth.heavy_tail_law(rng, H)
    qc, kc, vc = synth.calibration_samples(rng, kv, G, N)
    ref = O.calibrate_layer(qc, kc, vc, SIG)
    u_k, u_v, ck, cv = lib.calibrate_layer(qc, kc, vc, SIG, 0.999)
    for got, ref_bits, ref64 in ((u_k, ref["u_k"], ref["U_Q"]), (u_v, ref["u_v"], ref["U_S"])):
        g64 = O.bf16_to_f64(got)
        r64 = O.bf16_to_f64(ref_bits)
        # bf16 bits agree except where the fp64 value sits on a rounding tie
        diff = got != ref_bits
        assert diff.mean() < 1e-3, diff.mean()
        if diff.any():
            assert np.abs(g64 - r64)[diff].max() <= 2 ** -8 * np.abs(ref64)[diff].max()
    assert abs(float(ck) - float(ref["clip_k"])) <= 2e-7 * float(ref["clip_k"])
    assert abs(float(cv) - float(ref["clip_v"])) <= 2e-7 * float(ref["clip_v"])


def test_native_calibration_rejects_bad_arguments():
    with pytest.raises(lib.OscarError):
        lib.calibrate_layer(np.zeros((1, 1, 1, 128)), np.zeros((1, 1, 128)), np.zeros((1, 1, 128)), SIG)


@pytest.mark.parametrize("basis", ["identity", "naive", "calibrated"])
def test_native_clip_for_a_chosen_basis(basis):
    """oscar_calibrate_clip: the clip quantile of |x U H P| for any bf16 U, against
    the oracle's rotation and NumPy's linear-interpolation quantile; with the
    calibrated U it reproduces oscar_calibrate_layer's clip."""
    rng = np.random.default_rng(11)
    law = synth.outlier_law(rng, 2)
    qc, kc, vc = synth.calibration_samples(rng, law, 2, 400)
    if basis == "identity":
        u = O.f64_to_bf16(np.broadcast_to(np.eye(128), (2, 128, 128)))
    elif basis == "naive":
        # U = bf16(P H): R = U H P is the identity up to the bf16 rounding of U
        ph = O.bitrev_permutation() @ O.hadamard()
        u = O.f64_to_bf16(np.broadcast_to(ph, (2, 128, 128)))
        assert np.abs(O.rotation(u[0]) - np.eye(128)).max() < 2e-3
    else:
        u, _, ck, _ = lib.calibrate_layer(qc, kc, vc, SIG, 0.999)
        assert lib.calibrate_clip(kc, u) == ck
    want = np.quantile(np.concatenate([np.abs(kc[h] @ O.rotation(u[h])).ravel() for h in range(2)]), 0.999)
    got = float(lib.calibrate_clip(kc, u, 0.999))
    assert abs(got - want) <= 2e-7 * want
