"""The parity harness itself, on the CPU: compare() must pass what rounding
alone produces and fail on the mistakes the GPU tests exist to catch.

The mocks stand in for a GPU result.  They are the oracle's own outputs,
rounded as the kernels round, or the oracle run with a planted input-indexing
mistake (the batch-row class of unsloth-zoo PR #776, "What's changed": rows
past the first read or written at the wrong place), or with one (step, head)
row corrupted.
"""
import numpy as np
import pytest

from gated_delta_rule_recurrence_amd import inputs
from parity import OUTS, TOL, compare, row_errors, run_oracle

import oracle.gdr_oracle as O


def _problem(dtype="f32"):
    return inputs.draw(3, 24, 2, 4, 16, 8, seed=3, normalised=True, S0_std=0.1,
                       dST_std=1.0, dtype=dtype)


def _as_kernel_output(ref, dtype):
    """Round the oracle's outputs to what the kernels hand back: fp32 for the
    state-side tensors, the input dtype for the rest."""
    out = {}
    for n, a in ref.items():
        a32 = np.asarray(a, np.float32).astype(np.float64)
        out[n] = inputs.bf16_round(a32) if dtype == "bf16" and n not in ("S_T", "dS0") else a32
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rounding_alone_passes(dtype):
    p = _problem(dtype)
    ref = run_oracle(p)
    compare(_as_kernel_output(ref, dtype), ref, TOL[dtype], f"rounded {dtype}")


def test_wrong_batch_stride_fails():
    """A kernel that reads batch row 0's inputs for every row."""
    p = _problem()
    ref = run_oracle(p)
    bad = _problem()
    for n in ("q", "k", "v", "g", "beta", "dy"):
        a = getattr(bad, n)
        a[1:] = a[:1]
    bad.S0[1:] = bad.S0[:1]
    bad.dST[1:] = bad.dST[:1]
    mock = _as_kernel_output(run_oracle(bad), "f32")
    with pytest.raises(AssertionError):
        compare(mock, ref, TOL["f32"], "batch stride 0")


@pytest.mark.parametrize("name", ["dq", "dk", "dv", "dg", "dbeta", "dS0"])
def test_wrong_gradient_past_first_row_fails(name):
    """Gradients right for row 0 only: row 2 takes row 1's values."""
    p = _problem()
    ref = run_oracle(p)
    mock = _as_kernel_output(ref, "f32")
    mock[name] = mock[name].copy()
    mock[name][2] = mock[name][1]
    with pytest.raises(AssertionError):
        compare(mock, ref, TOL["f32"], f"{name} rows past the first")


def test_one_corrupted_row_fails_although_the_tensor_norm_passes():
    """One (step, value head) row of y zeroed out of 16,384 rows of a bf16
    output: the whole-tensor relative L2 stays under the bf16 bar (the
    rounding floor plus 1/sqrt(16384)), so only the per-row bound sees it."""
    rng = np.random.default_rng(5)
    ref = {"y": rng.standard_normal((1, 256, 64, 128))}
    mock = {"y": inputs.bf16_round(ref["y"])}
    mock["y"][0, 100, 17] = 0.0
    assert O.rel_l2(mock["y"], ref["y"]) <= TOL["bf16"]
    assert row_errors(mock["y"], ref["y"]).max() >= 0.99
    with pytest.raises(AssertionError, match="row"):
        compare(mock, ref, TOL["bf16"], "one zeroed row", names=("y",))


def test_one_wrong_scalar_gradient_fails():
    """One (step, value head) entry of dg with the wrong sign, in a bf16
    tensor of 16,384 entries; an entry of half the RMS, so that the
    whole-tensor error stays under the bar."""
    rng = np.random.default_rng(6)
    ref = {"dg": rng.standard_normal((1, 256, 64))}
    mock = {"dg": inputs.bf16_round(ref["dg"])}
    i = np.unravel_index(np.argmin(np.abs(np.abs(ref["dg"]) - 0.5)), ref["dg"].shape)
    mock["dg"][i] = -mock["dg"][i]
    assert O.rel_l2(mock["dg"], ref["dg"]) <= TOL["bf16"]
    with pytest.raises(AssertionError, match="row"):
        compare(mock, ref, TOL["bf16"], "one flipped dg entry", names=("dg",))


def test_non_finite_fails():
    p = _problem()
    ref = run_oracle(p)
    mock = _as_kernel_output(ref, "f32")
    mock["dS0"] = mock["dS0"].copy()
    mock["dS0"][0, 0, 0, 0] = np.nan
    with pytest.raises(AssertionError):
        compare(mock, ref, TOL["f32"], "nan")


def test_zero_reference_rows_are_held_absolutely():
    """Rows whose reference is exactly zero (masked steps' dv, dk) pass only
    if the result is zero to the tensor's own scale."""
    ref = {"dv": np.zeros((1, 4, 2, 8))}
    ref["dv"][0, 0] = 1.0
    ok = {"dv": ref["dv"].copy()}
    compare(ok, ref, TOL["f32"], "zero rows", names=("dv",))
    bad = {"dv": ref["dv"].copy()}
    bad["dv"][0, 3, 1, 2] = 1e-3
    with pytest.raises(AssertionError):
        compare(bad, ref, TOL["f32"], "zero rows", names=("dv",))


def test_outputs_covered():
    assert set(OUTS) == {"y", "S_T", "dq", "dk", "dv", "dg", "dbeta", "dS0"}
