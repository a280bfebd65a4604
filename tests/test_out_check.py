"""The output comparison of the GPU tests can see every term of the epilogue.

For every output check the GPU tests make (same case, threshold and sampled
outputs, from tests/parity_cases.py), the oracle's own output passes the
comparison, and the comparison rejects the oracle's output with one term of
"Core idea of LLM.int8()" step 3 or of the module's bias ("Class
Linear8bitLt", bias) done wrong:
  * the bias left out;
  * the bias applied per row (bias[t mod N]) instead of per output column;
  * the 16-bit outlier product left out.
A mutation that changes no element (no bias, a zero bias, N = 1 for the
per-row bias, no outlier column) is skipped: there is nothing to see.
"""
import numpy as np
import pytest

import oracle as O
from tests import parity_cases as PC
from tests.gpu_helpers import out_errors, out_ok

CHECKS = PC.output_checks()


def _oracle(case, tau, rows, cols):
    if isinstance(rows, str):  # the full-size config test's sample
        rows, cols = PC.config_sample(case)
    if cols is None:
        CB, SCB = O.quantize_weight_bits(case.W, case.dtype)
    else:  # only the sampled weight rows are read
        sCB, sSCB = O.quantize_weight_bits(case.W, case.dtype, rows=cols)
        CB = np.zeros((case.N, case.K), np.int8)
        SCB = np.zeros(case.N, np.float32)
        CB[cols], SCB[cols] = sCB, sSCB
    r = O.linear_forward(case.X, case.dtype, CB, SCB, case.bias, tau, rows=rows, cols=cols)
    rows_i = np.arange(case.T) if rows is None else np.asarray(rows)
    cols_i = np.arange(case.N) if cols is None else np.asarray(cols)
    SCBs = SCB[cols_i]
    D = O.dequantize(r["acc"], r["SCA"], SCBs)
    b = np.zeros(cols_i.size) if case.bias is None else O.decode_bits(case.bias, case.dtype).astype(np.float64)
    return r, D, b, rows_i, cols_i


@pytest.mark.parametrize("label,build,rows,cols", CHECKS, ids=[c[0] for c in CHECKS])
def test_checker_sees_every_epilogue_term(label, build, rows, cols):
    case, tau = build()
    r, D, b_full, rows_i, cols_i = _oracle(case, tau, rows, cols)
    dt = case.dtype
    nw, ratio = out_errors(r["out_bits"], r, dt)
    assert nw <= 1e-2 and ratio <= 1.0, f"the oracle's own rounded output: normwise {nw}, ratio {ratio}"

    e = r["out64"]
    b_col = b_full[cols_i][None, :] if case.bias is not None else np.zeros((1, cols_i.size))
    outlier = e - D - b_col
    mutations = {"bias dropped": e - b_col}
    if case.bias is not None:
        mutations["bias per row"] = e - b_col + b_full[rows_i % case.N][:, None]
    mutations["outlier product dropped"] = D + b_col
    seen = 0
    for what, m in mutations.items():
        if np.array_equal(m, e):
            continue  # changes nothing here
        assert not out_ok(O.round_to_dtype_bits(m, dt), r, dt), f"{what} passes the output check"
        seen += 1
    assert seen >= 1, "no term of the epilogue is visible in this case"
    if r["idx"].size and np.any(outlier != 0):
        assert not out_ok(O.round_to_dtype_bits(D + b_col, dt), r, dt)


def test_registry_covers_every_route_with_a_bias():
    """Every GPU output check with outliers on a biased case is in the registry
    with its bias: the random cases draw it N(0, 0.5), the size of an output."""
    labels = [c[0] for c in CHECKS]
    assert len(labels) == len(set(labels))
    case, _ = dict((c[0], c[1]) for c in CHECKS)["shape2000x768x4100-f16"]()
    b = O.decode_bits(case.bias, case.dtype)
    assert 0.3 < float(np.std(b)) < 0.7
