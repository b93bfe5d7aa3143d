"""gdr_forward_noalloc (the forward without a caller workspace: its per-chunk
records in the library's device scratch array) against gdr_forward, through
the C ABI, on two calls in a row: the Qwen3.5-9B heads at T=2048 (bf16, the
largest records of the two), then a smaller fp32 problem with an initial
state and a step mask, which reuses the array the first call left filled.
Both calls must give bitwise the same y, S_T and save buffer as gdr_forward
on the same inputs (the same kernels run on the same data), and the second
is also held to the oracle."""
import numpy as np
import pytest

from gated_delta_rule_recurrence_amd import _lib, inputs, ops
from parity import TOL, device_inputs, log

pytestmark = pytest.mark.gpu


def _run(p, dev, chunk, noalloc):
    import torch
    d = device_inputs(p, dev)
    mask = None
    if p.mask is not None:
        mask = torch.from_numpy(np.ascontiguousarray(p.mask, np.uint8)).to(dev)
    shape = ops.shape_of(d["q"], d["v"], chunk, d["q"].dtype)
    y = torch.full_like(d["v"], float("nan"))
    S_T = torch.full((p.B, p.Hv, p.Dv, p.Dk), float("nan"), dtype=torch.float32, device=dev)
    ckpt = torch.zeros(_lib.checkpoint_bytes(shape), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ptr = lambda t: 0 if t is None else t.data_ptr()
    args = [ptr(d[n]) for n in ("q", "k", "v", "g", "beta")] + [ptr(d["S0"])]
    if noalloc:
        st = _lib.forward_noalloc_raw(shape, *args, ptr(y), ptr(S_T), ptr(ckpt), stream,
                                      mask=ptr(mask))
    else:
        nws = _lib.forward_workspace_bytes(shape)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        st = _lib.forward_raw(shape, *args, ptr(y), ptr(S_T), ptr(ckpt), ptr(ws), nws,
                              stream, mask=ptr(mask))
    _lib.check(st, "gdr_forward_noalloc" if noalloc else "gdr_forward")
    torch.cuda.synchronize()
    return {"y": y.float().cpu().numpy(), "S_T": S_T.cpu().numpy(),
            "ckpt": ckpt.cpu().numpy()}


def test_noalloc_matches_forward_twice(cuda):
    import oracle.gdr_oracle as O
    big = inputs.qwen35_9b(2048)
    small = inputs.draw(2, 300, 2, 4, 64, 32, seed=71, normalised=True, S0_std=0.1,
                        decay="mix")
    rng = np.random.default_rng(71)
    small.mask = (rng.random((small.B, small.T)) >= 0.2).astype(np.uint8)
    for label, p, chunk in (("qwen T=2048 bf16", big, 64), ("small fp32 masked", small, 32)):
        log(f"noalloc vs gdr_forward: {label}")
        a = _run(p, cuda, chunk, noalloc=True)
        b = _run(p, cuda, chunk, noalloc=False)
        for n in a:
            np.testing.assert_array_equal(a[n], b[n], err_msg=f"{label}: {n}")
    y_ref, ST_ref = O.forward(small.q, small.k, small.v, small.g, small.beta, small.S0,
                              mask=small.mask)
    assert O.rel_l2(a["y"], y_ref) <= TOL["f32"]
    assert O.rel_l2(a["S_T"], ST_ref) <= TOL["f32"]


def test_noalloc_wide_keys(cuda):
    """Dk = 256 with bf16 inputs takes the chunked forward with 256-column
    tiles, whose records also go to the scratch array: bitwise gdr_forward's
    y, S_T and save buffer (a ragged last tile, S0 given)."""
    p = inputs.draw(1, 300, 4, 16, 256, 128, seed=91, normalised=True, S0_std=0.1,
                    decay="mix", dtype="bf16")
    shape = _lib.make_shape(1, 300, 4, 16, 256, 128, 64, _lib.GDR_BF16, 0)
    assert 0 < _lib.forward_workspace_bytes(shape) <= _lib.NOALLOC_SCRATCH_BYTES
    log("noalloc vs gdr_forward: Dk=256 bf16")
    a = _run(p, cuda, 64, noalloc=True)
    b = _run(p, cuda, 64, noalloc=False)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=f"Dk=256: {n}")
