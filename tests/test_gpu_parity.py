"""GPU parity of the HIP path (through the C ABI) against the float64
oracle, element by element on the same seeded inputs.

Bars: relative L2 <= 1e-5 on every output for fp32 inputs, <= 1e-2 for bf16
inputs against the oracle fed the same bf16-rounded inputs (the rel() metric
of mlx issue #4614).  Sizes span several tiles and ragged tails; the
Qwen3.5-9B shape at T=2048 (the benchmark's workload and launch
configuration) and the long-context shape are checked on sampled (batch row,
kv group) slices that the oracle computes on their own.
"""
import numpy as np
import pytest

from gated_delta_rule_recurrence_amd import inputs
from parity import (TOL, compare, compare_groups, device_inputs, log, run_gpu, run_oracle,
                    slice_group)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- config 1
@pytest.mark.parametrize("with_dST", [False, True])
@pytest.mark.parametrize("chunk", [1, 2, 3, 64])
def test_toy(cuda, with_dST, chunk):
    p = inputs.toy(seed=0, with_dST=with_dST)
    log(f"toy dST={with_dST} C={chunk}")
    compare(run_gpu(p, cuda, chunk), run_oracle(p), TOL["f32"], "toy")


# ---------------------------------------------------------------- config 2
@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_batch_rows(cuda, B):
    p = inputs.batch_rows(B)
    log(f"batch B={B}")
    gpu = run_gpu(p, cuda, 16)
    ref = run_oracle(p)
    compare(gpu, ref, TOL["f32"], f"B={B}")
    for b in range(1, B):  # rows past the first (unsloth-zoo PR #776)
        sl = {n: (a[b:b + 1]) for n, a in gpu.items()}
        rf = {n: (a[b:b + 1]) for n, a in ref.items()}
        compare(sl, rf, TOL["f32"], f"B={B} row {b}")


def test_batch_rows_bitwise_independent(cuda):
    p8 = inputs.batch_rows(8)
    g8 = run_gpu(p8, cuda, 64)
    for b in (0, 3, 7):
        p1 = inputs.batch_rows(8)
        for n in ("q", "k", "v", "g", "beta", "dy"):
            setattr(p1, n, getattr(p8, n)[b:b + 1].copy())
        p1.B = 1
        g1 = run_gpu(p1, cuda, 64)
        for n in g1:
            np.testing.assert_array_equal(g8[n][b:b + 1], g1[n], err_msg=f"row {b} {n}")


# ---------------------------------------------------------------- config 3
@pytest.mark.parametrize("heads", [(16, 48), (16, 16), (4, 12)])
@pytest.mark.parametrize("normalised", [False, True])
def test_strong_decay(cuda, heads, normalised):
    p = inputs.strong_decay(*heads, normalised=normalised)
    log(f"strong decay Hk/Hv={heads} normalised={normalised} "
        f"mean log g={p.meta['mean_log_g']:.2f}")
    compare(run_gpu(p, cuda, 64), run_oracle(p), TOL["f32"], "strong")


# ------------------------------------------------------ log-decay input (f2)
@pytest.mark.parametrize("chunk", [64, 7])
def test_log_decay_strong(cuda, chunk):
    """g given as log g; dg returned as dL/dlog g (chunked path at C=64, the
    per-step sweeps at C=7)."""
    p = inputs.draw(1, 128, 4, 12, 128, 128, seed=0, decay="strong", log_decay=True)
    log(f"log decay strong C={chunk}")
    compare(run_gpu(p, cuda, chunk), run_oracle(p), TOL["f32"], f"log strong C={chunk}")


def test_log_decay_bf16(cuda):
    p = inputs.draw(2, 70, 2, 4, 64, 32, seed=19, normalised=True, S0_std=0.1,
                    dST_std=1.0, dtype="bf16", log_decay=True)
    compare(run_gpu(p, cuda, 32), run_oracle(p), TOL["bf16"], "log bf16")


def test_log_decay_matches_plain_path(cuda):
    """Same problem through both encodings: every output agrees, and the
    log path's dg is g times the plain path's."""
    pl = inputs.draw(1, 100, 2, 4, 48, 40, seed=23, normalised=True, S0_std=0.2,
                     dST_std=1.0, log_decay=True)
    pg = inputs.draw(1, 100, 2, 4, 48, 40, seed=23, normalised=True, S0_std=0.2,
                     dST_std=1.0)
    a = run_gpu(pl, cuda, 32)
    b = run_gpu(pg, cuda, 32)
    b["dg"] = b["dg"] * pg.g
    compare(a, b, 2e-6, "log vs plain")


def test_strong_decay_short_chunks(cuda):
    p = inputs.strong_decay(4, 12)
    compare(run_gpu(p, cuda, 7), run_oracle(p), TOL["f32"], "strong C=7")


# ---------------------------------------------------------------- config 4
def test_qwen_bf16_T256_full(cuda):
    p = inputs.qwen35_9b(256)
    log("qwen35-9b bf16 T=256 full oracle")
    compare(run_gpu(p, cuda, 64), run_oracle(p), TOL["bf16"], "qwen T=256")


@pytest.mark.parametrize("decay,seed,s0", [("weak", 31, None), ("strong", 32, None),
                                             ("mix", 33, 0.05)])
def test_bf16_state_outputs_fp32_accurate(cuda, decay, seed, s0):
    """With bf16 inputs the state stays fp32 and the bf16-product kernels split
    every fp32 operand exactly into three bf16 pieces, so the products keep
    fp32 accuracy.  The bf16 outputs only show that to bf16 rounding; the
    fp32 outputs S_T (forward sweep) and dS0 (reverse sweep) must meet the
    fp32 bar against the oracle fed the same bf16-rounded inputs."""
    p = inputs.draw(1, 256, 16, 64, 192, 128, seed=seed, normalised=True, decay=decay,
                    S0_std=s0, dST_std=1.0, dtype="bf16")
    log(f"bf16 Qwen shape T=256 decay={decay}: fp32 outputs at the fp32 bar")
    errs = compare(run_gpu(p, cuda, 64), run_oracle(p), TOL["bf16"], f"bf16 {decay}")
    for name in ("S_T", "dS0"):
        assert errs[name] <= TOL["f32"], f"bf16 {decay}: {name} rel L2 {errs[name]:.2e}"


def test_bf16_products_match_fp32_path(cuda):
    """The bf16-product kernels against the fp32-operand kernels on the same
    bf16-valued inputs (headline shape, T=256).  Both compute at fp32
    accuracy, so after rounding the fp32 path's outputs to bf16 only a few in
    10,000 elements differ (rounding-boundary flips: 1.4-4.9e-4 of them, rel
    L2 of the difference 0.9-4.4e-5 when written).  A loss of precision in
    the piece products would raise both several-fold; the bars leave a
    fourfold margin."""
    import dataclasses
    p = inputs.qwen35_9b(256)
    p32 = dataclasses.replace(p, dtype="f32")
    gb, gf = run_gpu(p, cuda, 64), run_gpu(p32, cuda, 64)
    for name in ("y", "dq", "dk", "dv", "dg", "dbeta"):
        a, ref = gb[name], inputs.bf16_round(gf[name])
        frac = float(np.mean(a != ref))
        rel = float(np.linalg.norm(a - ref) / np.linalg.norm(ref))
        log(f"  {name}: differing {frac:.2e}, rel L2 {rel:.2e}")
        assert frac <= 2e-3 and rel <= 2e-4, f"{name}: differing {frac:.2e}, rel L2 {rel:.2e}"


def test_qwen_f32_T256_all_groups(cuda):
    """The headline heads with fp32 inputs (fp32-operand kernels): every kv
    group at the fp32 bar."""
    p = inputs.qwen35_9b(256, dtype="f32")
    gpu = run_gpu(p, cuda, 64)
    compare_groups(gpu, p, TOL["f32"], "qwen f32 T=256")


def test_qwen_bf16_log_decay_mask_all_groups(cuda):
    """The log-decay input and the step mask (rows f2, f4) at the headline
    heads, bf16, T=512, with a trainable S0 and dS_T: every kv group."""
    p = inputs.draw(1, 512, 16, 64, 192, 128, seed=89, normalised=True, decay="mix",
                    S0_std=0.05, dST_std=1.0, dtype="bf16", log_decay=True)
    rng = np.random.default_rng(89)
    p.mask = (rng.random((1, 512)) >= 0.1).astype(np.uint8)
    gpu = run_gpu(p, cuda, 64)
    compare_groups(gpu, p, TOL["bf16"], "qwen log+mask T=512", state_tol=TOL["f32"])


def test_qwen_bf16_T2048_long_interval_bitwise(cuda):
    """The benchmark workload with C = 128 and 512 (tiles replayed in the
    backward) equals C = 64 bit for bit."""
    p = inputs.qwen35_9b(2048)
    ref = run_gpu(p, cuda, 64)
    for C in (128, 512):
        got = run_gpu(p, cuda, C)
        for n in ref:
            np.testing.assert_array_equal(got[n], ref[n], err_msg=f"C={C}: {n}")


@pytest.mark.parametrize("T", [512, 1024, 2048])
def test_qwen_bf16_all_groups(cuda, T):
    """Config 4 at T = 512, 1024 and 2048 (the lengths of the mlx-lm PR #1217
    Performance table; 2048 is the benchmark workload in the benchmark's
    launch configuration): every kv group against the oracle run on that
    group alone, the bf16 outputs at the bf16 bar and the fp32 outputs S_T
    and dS0 at the fp32 bar."""
    p = inputs.qwen35_9b(T)
    log(f"qwen35-9b bf16 T={T}: all 16 kv groups")
    gpu = run_gpu(p, cuda, 64)
    compare_groups(gpu, p, TOL["bf16"], f"qwen T={T}", state_tol=TOL["f32"])


def test_qwen_bf16_B2_sampled(cuda):
    """B=2 selects two rows per lane in the sweeps (B=1 one, B=4 four)."""
    p = inputs.qwen35_9b(96, B=2)
    gpu = run_gpu(p, cuda, 32)
    for b, hk in ((0, 3), (1, 12)):
        compare(slice_group(gpu, p, b, hk), run_oracle(p, b, hk), TOL["bf16"],
                f"qwen B=2 b{b} kv{hk}")


# ---------------------------------------------------------------- config 5
@pytest.mark.parametrize("C", [64, 512])
def test_long_context_per_row(cuda, C):
    """Config 5 (B=4, T=8192, trainable S0, mixed decay): one kv group of
    every batch row against the oracle (a different group per row), the fp32
    outputs S_T and dS0 at the fp32 bar; at C=64 (a state and the residuals
    per 64 steps saved) and C=512 (a state per 512 steps, the tiles replayed
    in the backward)."""
    p = inputs.long_context()
    log(f"long context B=4 T=8192 C={C}: one kv group per batch row")
    gpu = run_gpu(p, cuda, C)
    compare_groups(gpu, p, TOL["bf16"], "long", units=[(0, 0), (1, 7), (2, 10), (3, 15)],
                   state_tol=TOL["f32"])


def test_chunked_checkpoints_hold_states(cuda):
    """The chunked forward's saved checkpoints (C = 64 on the Qwen3.5-9B heads,
    bf16 inputs, nonzero S0, mixed decay) are the states S_{64 j} of the
    recurrence, for every kv group, at the fp32 bar."""
    import torch
    import oracle.gdr_oracle as O
    T, C = 256, 64
    p = inputs.draw(1, T, 16, 64, 192, 128, seed=61, normalised=True, decay="mix",
                    S0_std=0.05, dtype="bf16")
    res = run_gpu(p, cuda, C, want_saved=True)
    nch = T // C
    n = p.B * p.Hv * nch * p.Dv * p.Dk
    ck = res["_saved"].ckpt[: 4 * n].view(dtype=torch.float32)
    ck = ck.reshape(p.B, p.Hv, nch, p.Dv, p.Dk).double().cpu().numpy()
    rep = p.Hv // p.Hk
    for hk in range(p.Hk):
        hs = slice(hk * rep, (hk + 1) * rep)
        _, _, states = O.forward(p.q[:, :, hk:hk + 1], p.k[:, :, hk:hk + 1], p.v[:, :, hs],
                                 p.g[:, :, hs], p.beta[:, :, hs], p.S0[:, hs],
                                 keep_states=True)
        for j in range(nch):
            err = O.rel_l2(ck[:, hs, j], states[C * j])
            assert err <= TOL["f32"], f"kv{hk} checkpoint {j}: rel L2 {err:.2e}"
    log(f"  checkpoints of {p.Hk} kv groups x {nch} chunks within {TOL['f32']}")


# ---------------------------------------------------------------- properties
def test_deterministic(cuda):
    p = inputs.strong_decay(4, 12)
    d = device_inputs(p, cuda)
    a = run_gpu(p, cuda, 64, d)
    b = run_gpu(p, cuda, 64, d)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)


def test_launch_events(cuda):
    """gdr_set_launch_events: a call records the caller's events right after
    its kernel launches, in order (forward: prep, sweep; backward on a grid
    small enough for head groups: prep, reverse sweep, chunk kernel, the sum
    of the groups' dq, dk terms); an event past a call's last launch is
    recorded at its end.  Every kernel's interval is positive, the extra one
    empty, the last event falls before an event recorded after the call, and
    the outputs are bit for bit those of a run without the hook."""
    import torch
    from gated_delta_rule_recurrence_amd import _lib, ops
    p = inputs.draw(1, 256, 2, 8, 128, 64, seed=101, normalised=True, S0_std=0.1,
                    dST_std=1.0, dtype="bf16")
    d = device_inputs(p, cuda)
    ref = run_gpu(p, cuda, 64, d)
    stream = torch.cuda.current_stream(cuda)
    ef = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    eb = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    end = torch.cuda.Event(enable_timing=True)
    for e in ef + eb + [end]:
        e.record(stream)  # creates the underlying events
    torch.cuda.synchronize()
    try:
        assert _lib.set_launch_events([e.cuda_event for e in ef[1:]]) == 0
        ef[0].record(stream)
        y, S_T, saved = ops.gdr_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"],
                                        chunk=64)
        assert _lib.set_launch_events([e.cuda_event for e in eb[1:]]) == 0
        eb[0].record(stream)
        outs = ops.gdr_backward(d["q"], d["k"], d["g"], d["beta"], saved, d["dy"], d["dST"])
        end.record(stream)
    finally:
        assert _lib.set_launch_events([]) == 0
    torch.cuda.synchronize()
    tf = [ef[i].elapsed_time(ef[i + 1]) for i in range(3)]
    tb = [eb[i].elapsed_time(eb[i + 1]) for i in range(4)]
    log(f"launch intervals ms: forward {tf}, backward {tb}")
    assert all(t > 0 for t in tf[:2] + tb), (tf, tb)
    assert 0 <= tf[2] < min(tf[:2]), tf  # past the forward's two launches
    assert eb[4].elapsed_time(end) >= 0
    got = dict(y=y, S_T=S_T, dq=outs[0], dk=outs[1], dv=outs[2], dg=outs[3], dbeta=outs[4],
               dS0=outs[5])
    for n, t in got.items():
        np.testing.assert_array_equal(t.float().cpu().numpy().astype(np.float64), ref[n],
                                      err_msg=f"with the hook: {n}")


def test_chunk_invariance(cuda):
    p = inputs.draw(2, 150, 2, 6, 64, 64, seed=5, normalised=True, S0_std=0.1,
                    dST_std=1.0)
    ref = run_gpu(p, cuda, 64)
    for C in (1, 7, 50, 128, 256):
        got = run_gpu(p, cuda, C)
        compare(got, ref, 2e-6, f"C={C} vs C=64")


def _masked(p, seed):
    rng = np.random.default_rng(seed)
    p.mask = (rng.random((p.B, p.T)) >= 0.2).astype(np.uint8)
    return p


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("C,tile", [(256, 64), (128, 64), (96, 48), (192, 64)])
def test_long_interval_replays_tiles_exactly(cuda, dtype, C, tile):
    """C > 64 saves a state every C steps only; the backward replays the
    tiles of each chunk from it with the same kernel, so every output equals
    the run with C = the tile bit for bit (ragged T, two batch rows, a mask,
    S0 and dS_T), and the oracle holds it to the bar."""
    p = _masked(inputs.draw(2, 300, 2, 4, 64, 32, seed=67, normalised=True, decay="mix",
                            S0_std=0.1, dST_std=1.0, dtype=dtype), 67)
    log(f"C={C} vs C={tile} {dtype}")
    a, b = run_gpu(p, cuda, C), run_gpu(p, cuda, tile)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=f"C={C} vs {tile}: {n}")
    compare(a, run_oracle(p), TOL[dtype], f"C={C} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_long_interval_replay_pair_grid(cuda, dtype):
    """Four value heads per kv head on a short sequence: the forward's prep
    runs one workgroup per pair of value heads, the backward's replay forms
    both record sets in one launch of eight one-wave heads; the records are
    the same element by element, so C = 128 still equals C = 64 bit for bit."""
    p = _masked(inputs.draw(2, 300, 2, 8, 64, 32, seed=73, normalised=True, decay="mix",
                            S0_std=0.1, dST_std=1.0, dtype=dtype), 73)
    log(f"C=128 vs C=64, Hv/Hk=4, {dtype}")
    a, b = run_gpu(p, cuda, 128), run_gpu(p, cuda, 64)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=f"C=128 vs 64: {n}")
    compare(a, run_oracle(p), TOL[dtype], f"C=128 Hv/Hk=4 {dtype}")


def test_long_interval_replay_without_segments(cuda):
    """More (batch row, saved state) pairs than one grid dimension holds: the
    replay runs every tile of a row from its first saved state instead of
    segment by segment; still bitwise the C=64 result."""
    B = 32768
    p = inputs.draw(B, 130, 1, 1, 16, 16, seed=71, normalised=True, S0_std=0.1)
    log(f"C=128 replay, B={B}")
    a, b = run_gpu(p, cuda, 128), run_gpu(p, cuda, 64)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)


@pytest.mark.parametrize("C", [100, 128])
def test_long_interval_per_step_path(cuda, C):
    """Dk = 200 takes the per-step sweeps; C=100 runs 50-step tiles, C=128
    64-step tiles, both replayed from states saved every C steps."""
    p = _masked(inputs.draw(2, 230, 1, 2, 200, 40, seed=73, normalised=True, decay="mix",
                            S0_std=0.1, dST_std=1.0), 73)
    log(f"per-step path C={C}")
    compare(run_gpu(p, cuda, C), run_oracle(p), TOL["f32"], f"per-step C={C}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_long_interval_decode(cuda, dtype):
    """T <= 8 with C > 64: one saved state (S0), replayed by the per-step sweep."""
    p = inputs.draw(3, 6, 2, 4, 192, 128, seed=79, normalised=True, S0_std=0.2,
                    dST_std=1.0, dtype=dtype)
    compare(run_gpu(p, cuda, 128), run_oracle(p), TOL[dtype], f"decode C=128 {dtype}")


def test_long_interval_saved_states(cuda):
    """At C = 128 the save buffer holds exactly the states S_{128 s}."""
    import torch
    import oracle.gdr_oracle as O
    p = inputs.draw(1, 300, 2, 4, 64, 32, seed=83, normalised=True, S0_std=0.1)
    res = run_gpu(p, cuda, 128, want_saved=True)
    nseg = 3
    ck = res["_saved"].ckpt.view(dtype=torch.float32)[: p.B * p.Hv * nseg * p.Dv * p.Dk]
    ck = ck.reshape(p.B, p.Hv, nseg, p.Dv, p.Dk).double().cpu().numpy()
    assert res["_saved"].ckpt.numel() == 4 * ck.size
    _, _, states = O.forward(p.q, p.k, p.v, p.g, p.beta, p.S0, keep_states=True)
    for j in range(nseg):
        assert O.rel_l2(ck[:, :, j], states[128 * j]) <= TOL["f32"], j


def test_gqa_matches_repeat_expanded(cuda):
    p = inputs.draw(1, 40, 2, 6, 32, 16, seed=9, normalised=True, S0_std=0.2)
    rep = p.Hv // p.Hk
    pe = inputs.draw(1, 40, 2, 6, 32, 16, seed=9, normalised=True, S0_std=0.2)
    pe.q = np.repeat(p.q, rep, axis=2)
    pe.k = np.repeat(p.k, rep, axis=2)
    pe.Hk = p.Hv
    a = run_gpu(p, cuda, 16)
    e = run_gpu(pe, cuda, 16)
    grp = lambda x: x.reshape(1, p.T, p.Hk, rep, -1).sum(3)
    e["dq"], e["dk"] = grp(e["dq"]), grp(e["dk"])
    compare(a, e, 1e-6, "gqa vs repeat")


def test_segment_chaining(cuda):
    """Two calls chained through S_T -> S0 and dS0 -> dS_T equal one call."""
    import torch
    from gated_delta_rule_recurrence_amd import ops
    p = inputs.draw(1, 90, 2, 4, 48, 40, seed=13, normalised=True, S0_std=0.1,
                    dST_std=1.0)
    d = device_inputs(p, cuda)
    y, ST, sv = ops.gdr_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], chunk=16)
    full = ops.gdr_backward(d["q"], d["k"], d["g"], d["beta"], sv, d["dy"], d["dST"])
    cut = 37
    A = {n: d[n][:, :cut].contiguous() for n in ("q", "k", "v", "g", "beta", "dy")}
    Bn = {n: d[n][:, cut:].contiguous() for n in ("q", "k", "v", "g", "beta", "dy")}
    y1, S1, sv1 = ops.gdr_forward(A["q"], A["k"], A["v"], A["g"], A["beta"], d["S0"], chunk=16)
    y2, S2, sv2 = ops.gdr_forward(Bn["q"], Bn["k"], Bn["v"], Bn["g"], Bn["beta"], S1, chunk=16)
    g2 = ops.gdr_backward(Bn["q"], Bn["k"], Bn["g"], Bn["beta"], sv2, Bn["dy"], d["dST"])
    g1 = ops.gdr_backward(A["q"], A["k"], A["g"], A["beta"], sv1, A["dy"], g2[5])
    torch.cuda.synchronize()
    np_ = lambda t: t.double().cpu().numpy()
    one = dict(y=y, S_T=ST, dq=full[0], dk=full[1], dv=full[2], dg=full[3],
               dbeta=full[4], dS0=full[5])
    two = dict(y=torch.cat([y1, y2], 1), S_T=S2, dq=torch.cat([g1[0], g2[0]], 1),
               dk=torch.cat([g1[1], g2[1]], 1), dv=torch.cat([g1[2], g2[2]], 1),
               dg=torch.cat([g1[3], g2[3]], 1), dbeta=torch.cat([g1[4], g2[4]], 1),
               dS0=g1[5])
    compare({k: np_(v) for k, v in two.items()}, {k: np_(v) for k, v in one.items()},
            2e-6, "chained")


@pytest.mark.parametrize("dims", [(5, 3), (36, 20), (100, 70), (256, 256), (130, 256)])
def test_ragged_and_max_dims(cuda, dims):
    Dk, Dv = dims
    p = inputs.draw(1, 45, 1, 2, Dk, Dv, seed=17, normalised=True, S0_std=0.2,
                    dST_std=1.0)
    log(f"dims Dk={Dk} Dv={Dv}")
    compare(run_gpu(p, cuda, 16), run_oracle(p), TOL["f32"], f"Dk={Dk} Dv={Dv}")


@pytest.mark.parametrize("B", [1, 2])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rows_per_lane_variants(cuda, B, dtype):
    """Wide heads (Hv=64, Dv=256) give the sweeps enough workgroups to hold 2
    (B=1) or 4 (B=2) state rows per lane on a 256-CU device; T=45 leaves a
    short last staging block after two full ones."""
    p = inputs.draw(B, 45, 16, 64, 16, 256, seed=37, normalised=True, S0_std=0.2,
                    dST_std=1.0, dtype=dtype)
    log(f"rows/lane B={B} {dtype}")
    compare(run_gpu(p, cuda, 16), run_oracle(p), TOL[dtype], f"wide B={B} {dtype}")


@pytest.mark.parametrize("Dk,chunk", [(256, 64), (232, 48), (248, 16)])
def test_bf16_wide_keys_chunked(cuda, Dk, chunk):
    """Dk above 192 with bf16 inputs runs the chunked sweeps with 256-column
    tiles (the E and C pieces overlaid on the q tile and on the gradient
    pieces, the prep's Gram products over Dk in two column passes): three
    32-row blocks, a ragged last tile, two batch rows, S0 and dS_T, mixed
    decay.  The bf16 outputs meet the bf16 bar and the fp32 outputs S_T, dS0
    the fp32 bar."""
    from gated_delta_rule_recurrence_amd import _lib
    p = inputs.draw(2, 150, 2, 4, Dk, 96, seed=79 + Dk, normalised=True, decay="mix",
                    S0_std=0.1, dST_std=1.0, dtype="bf16")
    sh = _lib.make_shape(2, 150, 2, 4, Dk, 96, chunk, _lib.GDR_BF16, 0)
    assert _lib.forward_workspace_bytes(sh) > 0, "not the chunked sweeps"
    log(f"bf16 wide keys Dk={Dk} chunk={chunk}")
    errs = compare(run_gpu(p, cuda, chunk), run_oracle(p), TOL["bf16"], f"bf16 Dk={Dk}")
    for name in ("S_T", "dS0"):
        assert errs[name] <= TOL["f32"], f"bf16 Dk={Dk}: {name} rel L2 {errs[name]:.2e}"


def test_bf16_wide_keys_full_grid(cuda):
    """Dk = 256 on a grid of 256 (tile, kv head, batch row) workgroups, so
    the chunk kernel runs one workgroup per kv head without head groups
    (T = 2048, 32 tiles); units of both batch rows against the oracle, the
    fp32 outputs at the fp32 bar."""
    from gated_delta_rule_recurrence_amd import _lib
    p = inputs.draw(2, 2048, 4, 8, 256, 64, seed=89, normalised=True, decay="mix",
                    S0_std=0.05, dST_std=1.0, dtype="bf16")
    sh = _lib.make_shape(2, 2048, 4, 8, 256, 64, 64, _lib.GDR_BF16, 0)
    assert _lib.forward_workspace_bytes(sh) > 0, "not the chunked sweeps"
    log("bf16 Dk=256 T=2048, 256 chunk workgroups")
    gpu = run_gpu(p, cuda, 64)
    compare_groups(gpu, p, TOL["bf16"], "Dk=256 T=2048", units=[(0, 0), (1, 3)],
                   state_tol=TOL["f32"])


def test_bf16_wide_keys_long(cuda):
    """Dk = 256 over 64 tiles (T = 4096, S0 and dS_T given, mixed decay):
    one unit against the oracle, the fp32 outputs at the fp32 bar."""
    p = inputs.draw(1, 4096, 2, 8, 256, 128, seed=97, normalised=True, decay="mix",
                    S0_std=0.05, dST_std=1.0, dtype="bf16")
    log("bf16 Dk=256 T=4096")
    gpu = run_gpu(p, cuda, 64)
    compare_groups(gpu, p, TOL["bf16"], "Dk=256 T=4096", units=[(0, 1)],
                   state_tol=TOL["f32"])


def test_bf16_wide_keys_replay(cuda):
    """C = 128 at Dk = 256: the backward's replay (the prep forming both
    record sets in one launch, the forward sweep in its general form) gives
    every output bit for bit as C = 64."""
    p = _masked(inputs.draw(2, 300, 2, 4, 256, 64, seed=83, normalised=True, decay="mix",
                            S0_std=0.1, dST_std=1.0, dtype="bf16"), 83)
    log("C=128 vs C=64, Dk=256 bf16")
    a, b = run_gpu(p, cuda, 128), run_gpu(p, cuda, 64)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=f"Dk=256 C=128 vs 64: {n}")
    compare(a, run_oracle(p), TOL["bf16"], "Dk=256 C=128")


@pytest.mark.parametrize("dims", [(72, 30), (68, 40), (136, 24), (192, 40), (64, 36),
                                  (192, 20), (104, 48), (128, 64), (56, 16), (200, 40),
                                  (256, 64), (252, 40), (250, 24)])
@pytest.mark.parametrize("chunk", [32, 64])
def test_bf16_dims(cuda, dims, chunk):
    """bf16 inputs at the edges of the bf16-product kernels' shape conditions
    (k rows in 8-element groups, value rows in 4-element blocks, dy rows in
    8-element blocks for the chunk-parallel part): Dk=72 with Dv=30 and Dk=68
    take the fp32-operand kernels, Dk=136 pads a 192-column tile, Dv=40 leaves
    a short last 32-row block, Dv=36 and Dv=20 pair the bf16-product sweeps
    with the fp32-operand chunk kernel; Dk=104 and 128 (128-column tiles) and
    56 (a 64-column tile) cover the other widths of the eight-wave chunk
    kernel, Dk=200 and 256 the 256-column tiles of the chunked sweeps and
    of the eight-wave chunk kernel; Dk=252 (4-element groups) and 250 take
    the per-step sweeps and the four-wave chunk kernel with bf16 inputs;
    T=70 leaves a short last chunk."""
    Dk, Dv = dims
    p = inputs.draw(1, 70, 2, 4, Dk, Dv, seed=23, normalised=True, S0_std=0.2,
                    dST_std=1.0, dtype="bf16")
    log(f"bf16 dims Dk={Dk} Dv={Dv} chunk={chunk}")
    compare(run_gpu(p, cuda, chunk), run_oracle(p), TOL["bf16"], f"bf16 Dk={Dk} Dv={Dv}")


@pytest.mark.parametrize("shape", [(4, 12, 72, 70), (2, 16, 64, 200), (1, 2, 32, 70)])
def test_bf16_head_groups(cuda, shape):
    """Short sequences whose (chunk, kv head, batch row) grid is under 256
    workgroups split each kv head's value heads over head groups, the dq, dk
    terms summed over the groups afterwards: 6 value heads per kv head in 3
    groups of 2 (96 workgroups before the split), 4 in 2 groups of 2 (128),
    and 16 in 16 groups of 1 (4)."""
    B, Hk, Hv, T = shape
    p = inputs.draw(B, T, Hk, Hv, 64, 32, seed=41, normalised=True, S0_std=0.2,
                    dST_std=1.0, dtype="bf16")
    log(f"bf16 head groups B={B} Hk={Hk} Hv={Hv} T={T}")
    compare(run_gpu(p, cuda, 64), run_oracle(p), TOL["bf16"], f"head groups {shape}")


def test_bf16_small(cuda):
    p = inputs.draw(2, 70, 2, 4, 64, 32, seed=19, normalised=True, S0_std=0.1,
                    dST_std=1.0, dtype="bf16")
    compare(run_gpu(p, cuda, 32), run_oracle(p), TOL["bf16"], "bf16 small")


def test_T1_and_empty(cuda):
    import torch
    from gated_delta_rule_recurrence_amd import ops
    p = inputs.draw(1, 1, 1, 2, 8, 8, seed=23, S0_std=0.5, dST_std=1.0)
    compare(run_gpu(p, cuda, 64), run_oracle(p), TOL["f32"], "T=1")
    # T = 0: S_T = S0 and dS0 = dS_T
    p0 = inputs.draw(1, 0, 1, 2, 8, 8, seed=23, S0_std=0.5, dST_std=1.0)
    d = device_inputs(p0, cuda)
    y, ST, sv = ops.gdr_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    grads = ops.gdr_backward(d["q"], d["k"], d["g"], d["beta"], sv, d["dy"], d["dST"])
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(ST, d["S0"])
    assert torch.equal(grads[5], d["dST"])


# ------------------------------------------------------- step mask (f4)
def _with_mask(p, seed, frac=0.3):
    rng = np.random.default_rng(seed)
    p.mask = (rng.random((p.B, p.T)) >= frac).astype(np.uint8)
    p.mask[0, 0] = 0
    p.mask[-1, -1] = 0
    return p


@pytest.mark.parametrize("chunk", [64, 7])
def test_mask_strong_decay(cuda, chunk):
    """Identity steps through the chunked path (C=64) and the per-step sweeps
    (C=7), strong decay, several batch rows."""
    p = _with_mask(inputs.draw(2, 150, 2, 6, 64, 64, seed=43, decay="strong",
                               normalised=True, S0_std=0.2, dST_std=1.0), 1)
    log(f"mask strong C={chunk}")
    compare(run_gpu(p, cuda, chunk), run_oracle(p), TOL["f32"], f"mask C={chunk}")


def test_mask_decode_and_bf16(cuda):
    p = _with_mask(inputs.draw(3, 5, 2, 4, 192, 128, seed=47, normalised=True,
                               S0_std=0.2, dST_std=1.0), 2)
    compare(run_gpu(p, cuda, 64), run_oracle(p), TOL["f32"], "mask decode")
    p = _with_mask(inputs.draw(2, 70, 2, 4, 64, 32, seed=53, normalised=True, S0_std=0.1,
                               dST_std=1.0, dtype="bf16", log_decay=True), 3)
    compare(run_gpu(p, cuda, 32), run_oracle(p), TOL["bf16"], "mask bf16 log")


def test_mask_variable_lengths(cuda):
    """A batch of sequences of unequal lengths, right- and left-padded in one
    call, against each sequence run alone (no mask) on the GPU."""
    import torch
    from gated_delta_rule_recurrence_amd import ops
    lens = [90, 41, 64, 17]
    T = max(lens)
    p = inputs.draw(len(lens), T, 2, 4, 96, 64, seed=59, normalised=True, S0_std=0.2,
                    dST_std=1.0)
    mask = np.zeros((p.B, T), np.uint8)
    for b, n in enumerate(lens):
        if b % 2 == 0:
            mask[b, :n] = 1          # right padding
        else:
            mask[b, T - n:] = 1      # left padding
    p.mask = mask
    for n_ in ("dy",):
        getattr(p, n_)[mask == 0] = 0.0  # no cotangent on padding
    full = run_gpu(p, cuda, 32)
    for b, n in enumerate(lens):
        keep = np.flatnonzero(mask[b])
        one = inputs.draw(1, 1, 2, 4, 96, 64, seed=0)  # shape holder
        for name in ("q", "k", "v", "g", "beta", "dy"):
            setattr(one, name, getattr(p, name)[b:b + 1][:, keep].copy())
        one.T = n
        one.S0 = p.S0[b:b + 1].copy()
        one.dST = p.dST[b:b + 1].copy()
        alone = run_gpu(one, cuda, 32)
        got = {k_: (v_[b:b + 1] if k_ in ("S_T", "dS0") else v_[b:b + 1][:, keep])
               for k_, v_ in full.items() if not k_.startswith("_")}
        compare(got, alone, 2e-6, f"varlen b{b} n={n}")


# ------------------------------------------- short sequences and decode (f3)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 3, 8])
def test_decode_steps(cuda, T, dtype):
    """T <= 8 takes the decode kernel; forward and backward (from its save
    buffer) against the oracle, several batch rows, Qwen3.5-9B head dims."""
    p = inputs.draw(3, T, 2, 4, 192, 128, seed=29, normalised=True, S0_std=0.2,
                    dST_std=1.0, dtype=dtype)
    log(f"decode T={T} {dtype}")
    compare(run_gpu(p, cuda, 64), run_oracle(p), TOL[dtype], f"decode T={T} {dtype}")


@pytest.mark.parametrize("dims", [(5, 3), (130, 20), (256, 256), (64, 17)])
def test_decode_ragged_dims(cuda, dims):
    Dk, Dv = dims
    p = inputs.draw(2, 2, 1, 2, Dk, Dv, seed=31, normalised=True, S0_std=0.2,
                    dST_std=1.0)
    compare(run_gpu(p, cuda, 1), run_oracle(p), TOL["f32"], f"decode Dk={Dk} Dv={Dv}")


def test_decode_in_place_state(cuda):
    """Inference with the state in and out of one buffer: T single-step calls
    with S_T = S0 (no save buffer) give the y and final state of one T-step
    call of the oracle."""
    import torch
    import oracle.gdr_oracle as O
    from gated_delta_rule_recurrence_amd import ops
    from parity import to_dev
    T = 6
    p = inputs.draw(2, T, 2, 4, 192, 128, seed=37, normalised=True, S0_std=0.2,
                    dtype="bf16")
    d = device_inputs(p, cuda)
    S = d["S0"].clone()
    ys = []
    for t in range(T):
        sl = {n: d[n][:, t:t + 1].contiguous() for n in ("q", "k", "v", "g", "beta")}
        y, _, saved = ops.gdr_forward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], S,
                                      save=False, S_T=S)
        assert saved is None
        ys.append(y)
    torch.cuda.synchronize()
    y_ref, S_ref = O.forward(p.q, p.k, p.v, p.g, p.beta, p.S0)
    got = torch.cat(ys, 1).float().cpu().numpy()
    assert O.rel_l2(got, y_ref) <= TOL["bf16"]
    assert O.rel_l2(S.cpu().numpy(), S_ref) <= 1e-5


def test_prefill_then_decode(cuda):
    """Prefill (chunked path, no save) then decode steps, state in place."""
    import torch
    import oracle.gdr_oracle as O
    from gated_delta_rule_recurrence_amd import ops
    T0, T1 = 100, 4
    p = inputs.draw(1, T0 + T1, 2, 4, 64, 48, seed=41, normalised=True, S0_std=0.1)
    d = device_inputs(p, cuda)
    S = d["S0"].clone()
    pre = {n: d[n][:, :T0].contiguous() for n in ("q", "k", "v", "g", "beta")}
    y0, _, _ = ops.gdr_forward(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], S,
                               save=False, S_T=S)
    ys = [y0]
    for t in range(T0, T0 + T1):
        sl = {n: d[n][:, t:t + 1].contiguous() for n in ("q", "k", "v", "g", "beta")}
        y, _, _ = ops.gdr_forward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], S,
                                  save=False, S_T=S)
        ys.append(y)
    torch.cuda.synchronize()
    y_ref, S_ref = O.forward(p.q, p.k, p.v, p.g, p.beta, p.S0)
    assert O.rel_l2(torch.cat(ys, 1).cpu().numpy(), y_ref) <= 1e-5
    assert O.rel_l2(S.cpu().numpy(), S_ref) <= 1e-5


def test_checkpoints_hold_states(cuda):
    """The saved state checkpoints are S_{jC} of the recurrence."""
    import oracle.gdr_oracle as O
    p = inputs.draw(1, 20, 1, 2, 16, 8, seed=29, normalised=True, S0_std=0.3)
    res = run_gpu(p, cuda, 6, want_saved=True)
    ck = res["_saved"].ckpt[: 4 * 4 * 2 * 8 * 16].view(dtype=__import__("torch").float32)
    ck = ck.reshape(1, 2, 4, 8, 16).double().cpu().numpy()
    _, _, states = O.forward(p.q, p.k, p.v, p.g, p.beta, p.S0, keep_states=True)
    for j in range(4):
        assert O.rel_l2(ck[:, :, j], states[6 * j]) <= 1e-6


@pytest.mark.parametrize("chunk", [8, 128])
def test_autograd_function(cuda, chunk):
    import torch
    from gated_delta_rule_recurrence_amd import ops
    p = inputs.draw(1, 133, 2, 4, 32, 16, seed=31, normalised=True, S0_std=0.1)
    d = device_inputs(p, cuda)
    leaves = [d[n].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "beta", "S0")]
    y, ST = ops.gated_delta_rule(*leaves, chunk=chunk)
    (y * d["dy"]).sum().backward()
    ref = run_oracle(p)
    import oracle.gdr_oracle as O
    for leaf, name in zip(leaves, ("dq", "dk", "dv", "dg", "dbeta", "dS0")):
        err = O.rel_l2(leaf.grad.double().cpu().numpy(), ref[name])
        assert err <= 1e-5, (name, err)
