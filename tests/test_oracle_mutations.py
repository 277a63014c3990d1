"""Plant plausible mistakes in a copy of the oracle; some pin must catch each.

The mistakes are planted in the oracle's source text on the CPU (a flipped bit
order, interleaved instead of contiguous groups, a transposed operand, an
averaged instead of summed gradient, ...). A mutation that no pin catches
would mean the pins do not fix that part of the oracle.
"""
import importlib.util
import os
import types

import pytest

from pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "sketch_oracle.py")

MUTATIONS = {
    "big_endian_bits": ('bitorder="little"', 'bitorder="big"'),
    "msb_first_fields": ("weights = (1 << np.arange(b, dtype=np.int64))",
                         "weights = (1 << np.arange(b, dtype=np.int64)[::-1])"),
    "interleaved_groups": ("return np.arange(d, dtype=np.int64) // (d // gpr)",
                           "return np.arange(d, dtype=np.int64) % gpr"),
    "reversed_groups": ("return lut[rows, g[None, :], idx]", "return lut[rows, (gpr - 1 - g)[None, :], idx]"),
    "index_off_by_one": ("return lut[rows, g[None, :], idx]",
                         "return lut[rows, g[None, :], (idx + 1) % lut.shape[2]]"),
    "forward_transposed": ("return X @ W.T", "return X @ W"),
    "forward_dropped_group": ("return X @ W.T", "return X[:, : W.shape[1] // 2] @ W[:, : W.shape[1] // 2].T"),
    "dx_sign": ("return dY @ W", "return -(dY @ W)"),
    "dx_transposed": ("return dY @ W", "return dY @ W.T"),
    "dw_transposed": ("return np.asarray(dY, dtype=np.float64).T @ np.asarray(X, dtype=np.float64)",
                      "return (np.asarray(X, dtype=np.float64).T @ np.asarray(dY, dtype=np.float64)).T[:, ::-1]"),
    "multi_set_ignored": ("W = dequantize(idx_packed, luts[int(lut_set[t])], d, b, gpr)",
                          "W = dequantize(idx_packed, luts[0], d, b, gpr)"),
    "multi_set_of_next_token": ("W = dequantize(idx_packed, luts[int(lut_set[t])], d, b, gpr)",
                                "W = dequantize(idx_packed, luts[int(lut_set[(t + 1) % m])], d, b, gpr)"),
    "adam_no_bias_correction": ("m_hat = m / (1.0 - beta1 ** step)", "m_hat = m"),
    "adam_bias_correction_power": ("v_hat = v / (1.0 - beta2 ** step)", "v_hat = v / (1.0 - beta2 ** (step + 1))"),
    "adam_swapped_betas": ("m = beta1 * np.asarray(exp_avg, dtype=np.float64) + (1.0 - beta1) * g",
                           "m = beta2 * np.asarray(exp_avg, dtype=np.float64) + (1.0 - beta2) * g"),
    "adam_eps_inside_sqrt": ("p = p - lr * m_hat / (np.sqrt(v_hat) + eps)", "p = p - lr * m_hat / np.sqrt(v_hat + eps)"),
    "adam_coupled_decay": ("p = p * (1.0 - lr * weight_decay)", "g = g + weight_decay * p"),
    "adam_grad_scale_ignored": ("g = np.asarray(grad, dtype=np.float64) * grad_scale\n    m =",
                                "g = np.asarray(grad, dtype=np.float64)\n    m ="),
    "sgd_dampened_momentum": ("buf = momentum * prev + g", "buf = momentum * prev + (1.0 - momentum) * g"),
    "sgd_decay_sign": ("* grad_scale + weight_decay * p", "* grad_scale - weight_decay * p"),
    "lloyd_unweighted_mean": ("swx = np.bincount(a, weights=wt * x, minlength=k)",
                              "swx = np.bincount(a, weights=x, minlength=k) * (sw / np.maximum(np.bincount(a, minlength=k), 1))"),
    "lloyd_init_edges": ("(np.arange(k, dtype=np.float64) + 0.5)", "(np.arange(k, dtype=np.float64) + 1.0)"),
    "lloyd_empty_to_zero": ("new = np.where(sw > 0, swx / np.where(sw > 0, sw, 1.0), c)",
                            "new = np.where(sw > 0, swx / np.where(sw > 0, sw, 1.0), 0.0)"),
    "lloyd_one_step_short": ("    for it in range(iters):\n        a = np.argmin",
                             "    for it in range(max(iters - 1, 0)):\n        a = np.argmin"),
    "map_no_division": ("err = (w[:, j] - t[rows, a]) / U[j, j]", "err = (w[:, j] - t[rows, a])"),
    "map_sign": ("w[:, j + 1:] -= err[:, None] * U[j, j + 1:][None, :]",
                 "w[:, j + 1:] += err[:, None] * U[j, j + 1:][None, :]"),
    "map_transposed_factor": ("w[:, j + 1:] -= err[:, None] * U[j, j + 1:][None, :]",
                              "w[:, j + 1:] -= err[:, None] * U[j + 1:, j][None, :]"),
    "column_weights_rows": ("return 1.0 / np.sum(U * U, axis=0)", "return 1.0 / np.sum(U * U, axis=1)"),
    "hessian_not_inverted": ("Hinv = np.linalg.inv(H)", "Hinv = H"),
    "dlut_overwrite": ("out[i, g[j], idx[i, j]] += dW[i, j]", "out[i, g[j], idx[i, j]] = dW[i, j]"),
    "dlut_average": (
        "out[i] = np.bincount(g * k + idx[i], weights=dW[i], minlength=gpr * k).reshape(gpr, k)",
        "out[i] = (np.bincount(g * k + idx[i], weights=dW[i], minlength=gpr * k)"
        " / np.maximum(1, np.bincount(g * k + idx[i], minlength=gpr * k))).reshape(gpr, k)"),
    "rel_err_mean_error": ("num = float(np.max(np.abs(got - ref)))", "num = float(np.mean(np.abs(got - ref)))"),
    "rel_err_sum_reference": ("den = float(np.max(np.abs(ref)))", "den = float(np.sum(np.abs(ref)))"),
    "rel_err_error_abs_dropped": ("num = float(np.max(np.abs(got - ref)))", "num = float(np.max(got - ref))"),
    "rel_err_reference_abs_dropped": ("den = float(np.max(np.abs(ref)))", "den = float(np.max(ref))"),
    "rel_err_swapped": ("    return num / den", "    return den / num"),
    "rel_err_scale_from_got": ("den = float(np.max(np.abs(ref)))", "den = float(np.max(np.abs(got)))"),
    "rel_err_elementwise": ("    return num / den",
                            "    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-300)))"),
    "rel_err_zero_reference_passes": ('return 0.0 if num == 0.0 else float("inf")', "return 0.0"),
    "rel_err_no_shape_check": ("if got.shape != ref.shape:", "if got.ndim != ref.ndim and False:"),
}


def _load_mutant(old, new):
    text = open(SRC).read()
    assert old in text, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(old, new), SRC + "[mutant]", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name):
    mutant = _load_mutant(*MUTATIONS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception as e:  # AssertionError, or a shape error from the mistake
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches mutation {name}"


def test_unmutated_copy_passes():
    text = open(SRC).read()
    mod = types.ModuleType("oracle_copy")
    exec(compile(text, SRC, "exec"), mod.__dict__)
    for pin in ALL_PINS:
        pin(mod)
