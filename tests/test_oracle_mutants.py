"""The oracle's pins are strong enough to catch plausible mistakes.

Each mutant plants one mistake in a copy of the oracle's source (a dropped
term, a wrong sign, index or position, a transposed operand, a missing
weight), on the CPU; the copy replaces the oracle's functions wherever the pin
tests look them up, and at least one pin must then fail.  The unmutated oracle
passes every pin (test_oracle.py, test_train_oracle.py)."""
import inspect
import sys
import types

import pytest

import oracle
import oracle.qkmla_oracle as dec_mod
import oracle.qkmla_train_oracle as train_mod

sys.path.insert(0, __file__.rsplit("/", 1)[0])
import test_oracle as pins  # noqa: E402
import test_train_oracle as train_pins  # noqa: E402

# (what the mistake is, original text, mutated text) in oracle/qkmla_oracle.py
DECODE_MUTANTS = [
    ("RoPE rotation sign", "out[..., 0::2] = x0 * cos - x1 * sin",
     "out[..., 0::2] = x0 * cos + x1 * sin"),
    ("RoPE pairs swapped", "out[..., 1::2] = x0 * sin + x1 * cos",
     "out[..., 1::2] = x1 * sin + x0 * cos"),
    ("RoPE frequency exponent", "-2.0 * i / rope_dim", "-1.0 * i / rope_dim"),
    ("RMS over the sum instead of the mean", "np.mean(z * z, axis=-1, keepdims=True)",
     "np.sum(z * z, axis=-1, keepdims=True)"),
    ("eps outside the square root", "np.sqrt(np.mean(z * z, axis=-1, keepdims=True) + eps)",
     "np.sqrt(np.mean(z * z, axis=-1, keepdims=True)) + eps"),
    ("gamma dropped from RMSNorm", "return z * np.asarray(gamma, dtype=F64) / rms(z, eps)",
     "return z / rms(z, eps)"),
    ("heads interleaved over groups", "return (h * n_groups) // n_heads",
     "return h % n_groups"),
    ("RoPE query at position L", "qr_hat = rope(rmsnorm(qr, gamma_q_rope, eps), L - 1, base)",
     "qr_hat = rope(rmsnorm(qr, gamma_q_rope, eps), L, base)"),
    ("plain-MLA RoPE query at position 0", "qr_hat = rope(qr, L - 1, base)",
     "qr_hat = rope(qr, 0, base)"),
    ("RoPE term dropped", "tau * (q_hat @ k_hat.T + qr_hat @ k_rope_hat[t0:t1].T)",
     "tau * (q_hat @ k_hat.T)"),
    ("softmax scale dropped", "tau * (q_hat @ k_hat.T + qr_hat @ k_rope_hat[t0:t1].T)",
     "(q_hat @ k_hat.T + qr_hat @ k_rope_hat[t0:t1].T)"),
    ("RoPE key not normalised", "return rope(rmsnorm(kr, gamma_k_rope, eps), pos, base)",
     "return rope(kr, pos, base)"),
    ("token chunk one row short", "t1 = min(L, t0 + chunk)", "t1 = min(L, t0 + chunk - 1)"),
    ("every chunk takes the first chunk's RoPE keys",
     "qr_hat @ k_rope_hat[t0:t1].T)", "qr_hat @ k_rope_hat[0:t1 - t0].T)"),
    ("key normalised with the query gamma", "k_hat = rmsnorm(k, gamma_k, eps) if qk_norm else k",
     "k_hat = rmsnorm(k, gamma_q, eps) if qk_norm else k"),
    ("log-sum-exp without its shift", "return e / s, (m + np.log(s))[..., 0]",
     "return e / s, (np.log(s))[..., 0]"),
    ("value side through group 0's W^UV", "o[b, heads] = v_lat @ np.asarray(w_uv[g], dtype=F64)",
     "o[b, heads] = v_lat @ np.asarray(w_uv[0], dtype=F64)"),
    ("causal prefix one row short", "keep = max(P_i + 1, 0)", "keep = max(P_i, 0)"),
    ("alpha is the RMS, not its inverse", "alpha[:, g] = 1.0 / rms(k, eps)[:, 0]",
     "alpha[:, g] = rms(k, eps)[:, 0]"),
    ("absorbed weight without gamma_k",
     "gg = np.asarray(gamma_q, dtype=F64) * np.asarray(gamma_k, dtype=F64)",
     "gg = np.asarray(gamma_q, dtype=F64)"),
    ("default scale over d_c only", "return 1.0 / math.sqrt(head_dim + rope_dim)",
     "return 1.0 / math.sqrt(head_dim)"),
]

# in oracle/qkmla_train_oracle.py
TRAIN_MUTANTS = [
    ("causal mask lets a row see the next token", "diagonal=1)", "diagonal=2)"),
    ("query RoPE at position 0", "qr = _rope(qr, pos[:, None], base)",
     "qr = _rope(qr, 0 * pos[:, None], base)"),
    ("key gamma on the query", "qh, kh = _rmsnorm(q_c, gamma_q, eps), _rmsnorm(k, gamma_k, eps)",
     "qh, kh = _rmsnorm(q_c, gamma_k, eps), _rmsnorm(k, gamma_k, eps)"),
    ("heads interleaved over groups", "gmap = [(h * G) // H for h in range(H)]",
     "gmap = [h % G for h in range(H)]"),
    ("values through group 0's W^UV", 'v = torch.einsum("btr,grd->btgd", c, w_uv)',
     'v = torch.einsum("btr,grd->btgd", c, w_uv[:1].expand_as(w_uv))'),
    ("packed sequence offset not advanced", "        row += L\n", "        row += 0\n"),
]


def _mutant_module(mod, old, new):
    src = inspect.getsource(mod)
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    m = types.ModuleType(mod.__name__ + "_mutant")
    m.__file__ = mod.__file__
    exec(compile(src.replace(old, new), mod.__file__ + " (mutant)", "exec"), m.__dict__)
    return m


def _install(monkeypatch, mutant, targets):
    """Point every name the pins look up at the mutant's functions."""
    for name, obj in vars(mutant).items():
        if isinstance(obj, types.FunctionType) and obj.__module__ == mutant.__name__:
            for t in targets:
                if hasattr(t, name):
                    monkeypatch.setattr(t, name, obj)


def _decode_pins():
    n_abs = len(pins.TINY_SHAPES) + 12
    calls = [(pins.test_absorbed_equals_explicit, (c,)) for c in range(0, n_abs, 3)]
    for name, fn in vars(pins).items():
        if name.startswith("test_") and name != "test_absorbed_equals_explicit":
            calls.append((fn, ()))
    return calls


def _train_pins():
    from mla_latent_decode_amd.inputs import Shape
    calls = [(train_pins.test_each_row_is_a_decode_over_its_prefix, (train_pins.SMALL, True)),
             (train_pins.test_each_row_is_a_decode_over_its_prefix,
              (Shape(6, 3, 10, 4, 6, 3, "f32"), True)),
             (train_pins.test_future_tokens_do_not_change_earlier_rows, ()),
             (train_pins.test_one_token_closed_forms, ()),
             (train_pins.test_packed_sequences_equal_the_batched_form, ()),
             (train_pins.test_packed_rows_do_not_see_other_sequences, ())]
    return calls


def _first_failure(calls):
    for fn, args in calls:
        try:
            fn(*args)
        except Exception as e:  # noqa: BLE001 -- any failure of a pin is a catch
            return f"{fn.__name__}{args}: {type(e).__name__}"
    return None


@pytest.mark.parametrize("what,old,new", DECODE_MUTANTS, ids=[m[0] for m in DECODE_MUTANTS])
def test_decode_oracle_mutant_is_caught(monkeypatch, what, old, new):
    mutant = _mutant_module(dec_mod, old, new)
    _install(monkeypatch, mutant, [dec_mod, oracle, pins])
    caught = _first_failure(_decode_pins())
    assert caught, f"no pin caught the planted mistake: {what}"
    print(f"{what}: caught by {caught}")


@pytest.mark.parametrize("what,old,new", TRAIN_MUTANTS, ids=[m[0] for m in TRAIN_MUTANTS])
def test_train_oracle_mutant_is_caught(monkeypatch, what, old, new):
    mutant = _mutant_module(train_mod, old, new)
    _install(monkeypatch, mutant, [train_mod, train_pins])
    caught = _first_failure(_train_pins())
    assert caught, f"no pin caught the planted mistake: {what}"
    print(f"{what}: caught by {caught}")


def test_unmutated_oracle_passes_the_pin_sets():
    """The harness itself: with nothing planted, no pin in either set fails."""
    assert _first_failure(_decode_pins()) is None
    assert _first_failure(_train_pins()) is None
