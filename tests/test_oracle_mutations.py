"""Planted mistakes in the oracle (on the CPU) must each be caught by a pin.

Each case monkeypatches one plausible error into the oracle module and checks
that the corresponding pin test then fails."""
import subprocess
import sys

import numpy as np
import pytest

import oracle
import oracle.oscar_oracle as OO
import test_oracle_attention as TA
import test_oracle_quant as TQ
import test_oracle_rotation as TR
from golden_io import kv_write_spikes, quantizer_groups


def _patch(monkeypatch, name, value):
    """Replace an oracle function both in its module and in the package."""
    monkeypatch.setattr(OO, name, value)
    monkeypatch.setattr(oracle, name, value)


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_identity_instead_of_bit_reversal_is_caught(monkeypatch):
    monkeypatch.setattr(OO, "bitrev7", lambda i: np.asarray(i, np.int64))
    case = [c for c in kv_write_spikes() if c["kind"] == "K" and c["k"] == 5][0]
    assert _fails(TQ.test_kv_write_golden_spikes, case)


def test_unnormalised_hadamard_is_caught(monkeypatch):
    orig = OO.hadamard
    _patch(monkeypatch, "hadamard", lambda d=128: orig(d) * np.sqrt(d))
    assert _fails(TR.test_lemma_diagonal_equalisation)


def test_zero_point_at_max_is_caught(monkeypatch):
    orig = OO.quantize

    def q_max(w, group=64):
        codes, s16, z16, s_pre, z_pre, t = orig(w, group)
        seg = w.reshape(w.shape[:-1] + (w.shape[-1] // group, group))
        return codes, s16, OO.fp16_rne(seg.max(-1)), s_pre, z_pre, t
    _patch(monkeypatch, "quantize", q_max)
    case = [c for c in quantizer_groups() if c["name"] == "ramp"][0]
    assert _fails(TQ.test_quantizer_golden, case)


def test_missing_inverse_rotation_is_caught(monkeypatch):
    monkeypatch.setattr(OO, "rotation", lambda u: np.eye(128))
    assert _fails(TA.test_hand_built_int2_page_closed_form)


def test_swapped_k_v_code_layouts_are_caught(monkeypatch):
    monkeypatch.setattr(OO, "V_CODES", 0)
    monkeypatch.setattr(OO, "K_CODES", 512)
    assert _fails(TA.test_hand_built_int2_page_closed_form)


def test_oracle_imports_no_product_code():
    code = ("import sys, oracle, synth; "
            "bad=[m for m in sys.modules if m.startswith('int2_rotated_kv_write_amd') or m == 'torch']; "
            "print(bad); sys.exit(1 if bad else 0)")
    r = subprocess.run([sys.executable, "-c", code], cwd=TR.__file__.rsplit("/tests/", 1)[0],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
