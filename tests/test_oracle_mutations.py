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


def _extend_mutant(causal_end):
    """The oracle's extend with the chunk-key bound replaced (t0 .. causal_end(t, t1))."""
    def ext(shape, cache, layer, q_bits, k_bits, v_bits, cu_seqlens, prefix_lens, page_table, sm_scale):
        q, kn, vn = OO.bf16_to_f64(q_bits), OO.bf16_to_f64(k_bits), OO.bf16_to_f64(v_bits)
        T, Hq, _ = q.shape
        G = shape.gqa
        out = np.zeros((T, Hq, OO.D))
        for b in range(len(cu_seqlens) - 1):
            t0, t1, L = int(cu_seqlens[b]), int(cu_seqlens[b + 1]), int(prefix_lens[b])
            for h in range(shape.num_kv_heads):
                Kp, Vp, _ = OO.gather_sequence(shape, cache, layer, b, h, L, page_table)
                for t in range(t0, t1):
                    e = causal_end(t, t1)
                    K, V = np.concatenate([Kp, kn[t0:e, h]]), np.concatenate([Vp, vn[t0:e, h]])
                    for hq in range(h * G, (h + 1) * G):
                        lg = sm_scale * (K @ q[t, hq])
                        p = np.exp(lg - lg.max())
                        out[t, hq] = (p @ V) / p.sum()
        return out
    return ext


def test_extend_without_causal_mask_is_caught(monkeypatch):
    import test_oracle_extend as TE
    _patch(monkeypatch, "extend", _extend_mutant(lambda t, t1: t1))
    assert _fails(TE.test_bf16_only_prefix_equals_brute_force_causal, 10, 7)


def test_extend_excluding_its_own_key_is_caught(monkeypatch):
    import test_oracle_extend as TE
    _patch(monkeypatch, "extend", _extend_mutant(lambda t, t1: t))
    assert _fails(TE.test_bf16_only_prefix_equals_brute_force_causal, 10, 7)


def test_extend_with_a_short_prefix_is_caught(monkeypatch):
    import test_oracle_extend as TE
    orig = OO.gather_sequence
    monkeypatch.setattr(OO, "gather_sequence",
                        lambda shape, cache, layer, b, h, L, table: orig(shape, cache, layer, b, h, max(L - 1, 0), table))
    assert _fails(TE.test_bf16_only_prefix_equals_brute_force_causal, 150, 20)
