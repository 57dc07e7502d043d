"""HIP path vs the fp64 oracle, element by element, at sizes the oracle
finishes in seconds: the tiny fp32 workload, the 4096-token workload, and
ragged shapes spanning several tiles (256 tokens x 320 vocabulary columns in
the forward and the logit recompute; 256 x 256 in the dW and dH products, or
128 x 256 where 256 x 256 tiles would be fewer than the compute units) with
partial tails in every dimension; plus the degenerate cases of the method."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as WL
from oracle import compare as C
from tests.gpu_common import require_gpu, run_gpu, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vp():
    return require_gpu()


def full_check(vp, w: WL.Workload, seed=0, dloss=1.0, R=None):
    R = w.R if R is None else R
    say(f"case {w.name} N={w.N} d={w.d} V={w.V} R={R} {w.dtype} seed={seed}")
    inp = WL.make_inputs(w, seed)
    H, W, lab = to_device(inp)
    loss, lse, dH, dW = run_gpu(vp, H, W, lab, R, dloss=dloss)
    Hf, Wf = inp.H_f64(), inp.W_f64()
    rloss, rlse = oracle.forward(Hf, Wf, inp.labels)
    rdH, rdW = oracle.backward(Hf, Wf, inp.labels, dloss)
    e_lse = C.lse_err(lse, rlse)
    e_loss = C.loss_rel_err(loss, rloss)
    okH, eH = C.grad_ok(dH, rdH)
    okW, eW = C.grad_ok(dW, rdW)
    say(C.report(w.name, lse=e_lse, loss=e_loss, dH_maxabs=eH[0],
                 dH_ref=eH[1], dH_cos=eH[2], dW_maxabs=eW[0], dW_ref=eW[1],
                 dW_cos=eW[2]))
    assert e_lse <= C.LSE_ABS, e_lse
    assert e_loss <= C.LOSS_REL, (loss, rloss)
    assert okH, eH
    assert okW, eW
    ign = inp.labels == -100
    assert np.all(dH[ign] == 0.0)
    return loss, lse, dH, dW


def test_tiny_f32_workload(vp):
    full_check(vp, WL.WORKLOADS[0])


def test_n4096_d2048_v32000_r4_workload(vp):
    full_check(vp, WL.WORKLOADS[1])


RAGGED = [
    # N, d, V, R, dtype
    (300, 136, 1000, 3, "bf16"),
    (257, 72, 515, 7, "bf16"),
    (513, 264, 2049, 2, "bf16"),
    (300, 136, 1000, 3, "f32"),
    (1, 8, 5, 5, "bf16"),
    (64, 64, 33, 33, "f32"),
    (700, 520, 4500, 1, "bf16"),
    (300, 64, 40000, 1, "bf16"),   # one shard over three backward chunks
                                   # (4 x 8192 + ragged 7232 columns)
    # shard widths at, above and below the 320-column vocabulary tile
    (260, 64, 640, 2, "bf16"),     # 320 + 320: whole tiles
    (300, 136, 963, 3, "bf16"),    # 321 each: a full tile and a 1-column one
    (257, 72, 1276, 4, "f32"),     # 319 each: one tile, last column empty
    (129, 96, 3841, 3, "bf16"),    # 1281 / 1280 / 1280: four tiles (+ 1)
]


@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "x".join(map(str, c)))
def test_ragged_shapes(vp, case):
    N, d, V, R, dt = case
    w = WL.custom(N, d, V, R, dtype=dt, w_std=0.3, ignore_frac=0.1,
                  name="ragged")
    full_check(vp, w, seed=7, dloss=0.75)


def test_product_tile_switch_at_the_compute_unit_count(vp):
    """The dH product runs on 128 x 256 tiles where 256 x 256 tiles would be
    fewer than the device's compute units (dW, whose operands are both read
    K-outer, always on 256 x 256 tiles, in the same launch). With d = 2048 (8
    column tiles) these two shapes put dH just below and just above that
    count and the dW grid just at / below it, so both launch variants meet
    the oracle, with ragged row tails."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = cus // 8                       # 256-row tiles for cus tiles
    cases = [
        # N: dH just below / above;  V = 2 * chunk: dW just at / below
        (256 * (rows - 1) - 100, 2 * (256 * rows - 192)),
        (256 * (rows + 1) - 100, 2 * (256 * (rows - 1) - 92)),
    ]
    for N, V in cases:
        dh_tiles = -(-N // 256) * 8
        dw_tiles = -(-(V // 2) // 256) * 8
        say(f"cus={cus} N={N} V={V}: dH tiles {dh_tiles}, dW tiles {dw_tiles}")
        assert (dh_tiles < cus) != (dw_tiles < cus)
        w = WL.custom(N=N, d=2048, V=V, R=2, w_std=0.02, ignore_frac=0.03,
                      name=f"switch_n{N}_v{V}")
        full_check(vp, w)


def test_outlier_rows_large_logits(vp):
    w = WL.custom(1000, 256, 3000, 3, w_std=0.05, ignore_frac=0.1,
                  outlier_frac=0.05, outlier_scale=20.0, labels="zipf",
                  zipf_s=1.2, name="outliers")
    full_check(vp, w, seed=3)


def test_shard_count_invariance_on_gpu(vp):
    w = WL.custom(512, 256, 5000, 1, w_std=0.1, ignore_frac=0.05)
    inp = WL.make_inputs(w, 11)
    H, W, lab = to_device(inp)
    say("case shard invariance R=1 vs R=8 vs R=7")
    res = {R: run_gpu(vp, H, W, lab, R) for R in (1, 8, 7)}
    for R in (8, 7):
        assert C.loss_rel_err(res[R][0], res[1][0]) <= 1e-5
        assert C.lse_err(res[R][1], res[1][1]) <= 1e-4
        assert C.grad_ok(res[R][2], res[1][2])[0]
        assert C.grad_ok(res[R][3], res[1][3])[0]


def test_zero_weights_give_log_v(vp):
    V = 1000
    w = WL.custom(300, 64, V, 3, w_std=0.0)
    inp = WL.make_inputs(w, 0)
    H, W, lab = to_device(inp)
    say("case W=0")
    loss, lse, dH, dW = run_gpu(vp, H, W, lab, 3)
    assert np.max(np.abs(lse - math.log(V))) < 2e-5
    assert abs(loss - math.log(V)) < 2e-5
    assert np.all(dH == 0.0)
    rdW = oracle.backward(inp.H_f64(), inp.W_f64(), inp.labels)[1]
    assert C.grad_ok(dW, rdW)[0]


def test_all_ignored(vp):
    w = WL.custom(200, 32, 300, 2, w_std=0.2)
    inp = WL.make_inputs(w, 0)
    inp.labels[:] = -100
    H, W, lab = to_device(inp)
    say("case all ignored")
    loss, lse, dH, dW = run_gpu(vp, H, W, lab, 2)
    assert loss == 0.0
    assert np.all(dH == 0.0) and np.all(dW == 0.0)
    rlse = oracle.forward(inp.H_f64(), inp.W_f64(), inp.labels)[1]
    assert C.lse_err(lse, rlse) <= C.LSE_ABS


def test_invalid_label_gives_nan_loss(vp):
    w = WL.custom(100, 32, 300, 2, w_std=0.2)
    inp = WL.make_inputs(w, 0)
    for bad in (300, -1, 1 << 40):
        inp.labels[5] = bad
        H, W, lab = to_device(inp)
        say(f"case invalid label {bad}")
        loss, lse = vp.forward(H, W, lab, 2)
        assert math.isnan(loss.item())
        assert torch.isfinite(lse).all()


def test_custom_ignore_index(vp):
    w = WL.custom(300, 64, 500, 2, w_std=0.3)
    inp = WL.make_inputs(w, 4)
    inp.labels[::7] = 499           # 499 is a real class used as ignore mark
    H, W, lab = to_device(inp)
    say("case ignore_index=499")
    loss, lse, dH, dW = run_gpu(vp, H, W, lab, 2, ignore_index=499)
    rloss, rlse = oracle.forward(inp.H_f64(), inp.W_f64(), inp.labels, 499)
    rdH, rdW = oracle.backward(inp.H_f64(), inp.W_f64(), inp.labels, 1.0, 499)
    assert C.loss_rel_err(loss, rloss) <= C.LOSS_REL
    assert C.lse_err(lse, rlse) <= C.LSE_ABS
    assert C.grad_ok(dH, rdH)[0] and C.grad_ok(dW, rdW)[0]


def test_empty_batch(vp):
    d, V = 64, 100
    H = torch.empty((0, d), dtype=torch.bfloat16, device="cuda")
    W = torch.randn((V, d), device="cuda").to(torch.bfloat16)
    lab = torch.empty(0, dtype=torch.int64, device="cuda")
    say("case N=0")
    loss, lse = vp.forward(H, W, lab, 4)
    dH, dW = vp.backward(H, W, lab, lse, None, 4)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and lse.numel() == 0
    assert dH.shape == (0, d) and torch.all(dW == 0)


def test_bitwise_determinism(vp):
    w = WL.custom(777, 136, 3000, 3, w_std=0.2, ignore_frac=0.05)
    inp = WL.make_inputs(w, 2)
    H, W, lab = to_device(inp)
    say("case determinism")
    a = run_gpu(vp, H, W, lab, 3, dloss=1.7)
    b = run_gpu(vp, H, W, lab, 3, dloss=1.7)
    assert a[0] == b[0]
    for x, y in zip(a[1:], b[1:]):
        assert np.array_equal(x, y)


def test_dloss_scaling_is_linear(vp):
    w = WL.custom(300, 64, 700, 2, w_std=0.2, ignore_frac=0.1)
    inp = WL.make_inputs(w, 5)
    H, W, lab = to_device(inp)
    say("case dloss scaling")
    a = run_gpu(vp, H, W, lab, 2, dloss=1.0)
    b = run_gpu(vp, H, W, lab, 2, dloss=-4.0)
    # exact up to bf16 storage of G near the denormal range
    for x, y in ((b[2], a[2]), (b[3], a[3])):
        np.testing.assert_allclose(x, -4.0 * y, rtol=1e-6,
                                   atol=1e-6 * np.abs(y).max())


def test_argument_errors_raise(vp):
    H = torch.zeros((8, 12), dtype=torch.bfloat16, device="cuda")  # d % 8
    W = torch.zeros((10, 12), dtype=torch.bfloat16, device="cuda")
    lab = torch.zeros(8, dtype=torch.int64, device="cuda")
    with pytest.raises(vp.VPCEError):
        vp.forward(H, W, lab, 1)
    H = torch.zeros((8, 16), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((10, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(vp.VPCEError):
        vp.forward(H, W, lab, 11)     # R > V
    with pytest.raises(vp.VPCEError):
        vp.forward(H, W, lab, 1, workspace=torch.empty(16, dtype=torch.uint8,
                                                       device="cuda"))


def test_workspace_is_independent_of_v(vp):
    """Peak device bytes minus inputs and outputs is the same for every V
    (the logit tensor never exists; only block-sized state does)."""
    N, d, R = 1024, 256, 4
    extra = []
    for V in (8000, 32000, 64000):
        H = torch.randn((N, d), device="cuda").to(torch.bfloat16)
        W = (torch.randn((V, d), device="cuda") * 0.05).to(torch.bfloat16)
        lab = torch.randint(0, V, (N,), device="cuda")
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        say(f"case V-sweep V={V}")
        loss, lse = vp.forward(H, W, lab, R)
        dH, dW = vp.backward(H, W, lab, lse, None, R)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated()
        outs = sum(t.numel() * t.element_size() for t in (loss, lse, dH, dW))
        extra.append(peak - base - outs)
        del H, W, lab, loss, lse, dH, dW
        torch.cuda.empty_cache()
    # the caching allocator may hand out a block up to 1 MiB larger than
    # requested; a V-sized buffer would differ by N*V*4 = 32..262 MB here
    ws = vp.workspace_bytes(N, d, 8000, R)
    slack = 2 << 20
    assert all(abs(e - extra[0]) <= slack for e in extra), extra
    assert all(e <= ws + slack for e in extra), (extra, ws)


def test_narrow_workspace_runs_ragged_chunks(vp):
    """A workspace sized for 768-column backward chunks: each 2500-wide shard
    runs as 768, 768, 768, 196. dW rows come out of one chunk each (bitwise
    equal to the full-width run); dH sums the chunks in another grouping."""
    w = WL.Workload("narrow_chunks", N=2048, d=256, V=5000, R=2, dtype="bf16",
                    w_std=0.05, labels="zipf", zipf_s=1.1, ignore_frac=0.03)
    say(f"case {w.name} N={w.N} d={w.d} V={w.V} R={w.R} chunk 768")
    inp = WL.make_inputs(w, 4)
    H, W, lab = to_device(inp)
    full = run_gpu(vp, H, W, lab, w.R)
    ws = torch.empty(vp.workspace_bytes(w.N, w.d, w.V, w.R, H.dtype,
                                        chunk_cols=768),
                     dtype=torch.uint8, device=H.device)
    assert ws.numel() < vp.workspace_bytes(w.N, w.d, w.V, w.R, H.dtype)
    loss, lse = vp.forward(H, W, lab, w.R, workspace=ws)
    dH, dW = vp.backward(H, W, lab, lse, None, w.R, workspace=ws)
    torch.cuda.synchronize()
    dH = dH.cpu().numpy().astype(np.float64)
    dW = dW.cpu().numpy().astype(np.float64)
    assert float(loss.item()) == full[0]
    assert np.array_equal(lse.cpu().numpy().astype(np.float64), full[1])
    assert np.array_equal(dW, full[3])
    assert np.abs(dH - full[2]).max() <= 1e-6 * np.abs(full[2]).max()
    Hf, Wf = inp.H_f64(), inp.W_f64()
    rdH, rdW = oracle.backward(Hf, Wf, inp.labels, 1.0)
    okH, eH = C.grad_ok(dH, rdH)
    okW, eW = C.grad_ok(dW, rdW)
    say(C.report(w.name, dH_maxabs=eH[0], dH_ref=eH[1], dH_cos=eH[2],
                 dW_maxabs=eW[0], dW_ref=eW[1], dW_cos=eW[2]))
    assert okH, eH
    assert okW, eW


def test_planned_peak_is_the_measured_peak(vp):
    """The planner's peak, known before launch, against the exact bytes the
    allocator handed out during one forward + backward (requested sizes,
    before the allocator's own rounding)."""
    N, d, V, R = 4096, 1024, 32000, 4
    fixed = (N * d * 2 + V * d * 2 + 8 * N) + (4 * N + 4 + 4 * N * d
                                               + 4 * V * d)
    budget = fixed + vp.workspace_bytes(N, d, V, R, torch.bfloat16,
                                        chunk_cols=2048)
    plan = vp.plan(N, d, V, R, budget)
    say(f"case planned peak N={N} d={d} V={V} R={R} plan={plan}")
    assert plan["chunk_cols"] == 2048 and plan["peak_bytes"] == budget
    torch.cuda.synchronize()
    base = torch.cuda.memory_stats()["requested_bytes.all.current"]
    g = torch.Generator(device="cuda").manual_seed(2)
    H = torch.randn((N, d), device="cuda", generator=g).to(torch.bfloat16)
    W = (torch.randn((V, d), device="cuda", generator=g) * 0.03).to(
        torch.bfloat16)
    lab = torch.randint(0, V, (N,), device="cuda", generator=g)
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    loss, lse = vp.forward(H, W, lab, R, workspace=ws)
    dH, dW = vp.backward(H, W, lab, lse, None, R, workspace=ws)
    torch.cuda.synchronize()
    peak = torch.cuda.memory_stats()["requested_bytes.all.peak"] - base
    say(f"planned {plan['peak_bytes']} measured {peak}")
    assert peak == plan["peak_bytes"]
    assert math.isfinite(float(loss.item()))


def test_seeded_random_shapes(vp):
    """Forty shapes drawn from a fixed seed: bf16 and fp32, N up to 3000, d
    up to 1600, V up to 6000, R from 1 to 9, none to half of the tokens
    ignored, three logit scales and upstream gradients; every one at oracle
    parity."""
    rng = np.random.default_rng(12345)
    for case in range(40):
        dt = "bf16" if rng.random() < 0.8 else "f32"
        mult = 8 if dt == "bf16" else 4
        N = int(rng.integers(1, 3000))
        d = int(rng.integers(1, 200)) * mult
        R = int(rng.integers(1, 10))
        V = int(rng.integers(R, 6000))
        ign = float(rng.choice([0.0, 0.05, 0.5]))
        w_std = float(rng.choice([0.02, 0.2, 3.0 / d ** 0.5]))
        dloss = float(rng.choice([1.0, 0.37, 2.5]))
        w = WL.custom(N=N, d=d, V=V, R=R, dtype=dt, w_std=w_std,
                      ignore_frac=ign, name=f"random{case}")
        full_check(vp, w, seed=case, dloss=dloss)


def test_traced_calls_match_and_bracket_every_launch(vp):
    """vpce_forward_traced / vpce_backward_traced: the same outputs as the
    untraced calls (bitwise), one event pair per kernel launch with its kind
    in launch order (forward: fill, tile kernel, merge, loss; backward: the
    gradient scale, then per chunk the recompute and the product launch),
    and every pair's elapsed time is non-negative."""
    N, d, V, R = 700, 136, 4500, 3      # shards 1500: one chunk each
    w = WL.custom(N=N, d=d, V=V, R=R, w_std=0.3, ignore_frac=0.05,
                  name="traced")
    inp = WL.make_inputs(w, 17)
    H, W, lab = to_device(inp)
    say(f"case traced calls N={N} d={d} V={V} R={R}")
    loss0, lse0 = vp.forward(H, W, lab, R)
    dH0, dW0 = vp.backward(H, W, lab, lse0, None, R)

    def events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for e in evs:
            e.record()
        return evs

    fe, be = events(8), events(16)
    loss, lse, kf, nf = vp.forward_traced(H, W, lab, R, fe)
    dH, dW, kb, nb = vp.backward_traced(H, W, lab, lse, None, R, be)
    torch.cuda.synchronize()
    assert kf == ["other", "forward_tile", "merge", "other"] and nf == 4
    assert kb == ["other"] + ["recompute", "products"] * R and nb == 1 + 2 * R
    for evs, n in ((fe, nf), (be, nb)):
        for i in range(n):
            assert evs[2 * i].elapsed_time(evs[2 * i + 1]) >= 0.0
    assert torch.equal(loss, loss0) and torch.equal(lse, lse0)
    assert torch.equal(dH, dH0) and torch.equal(dW, dW0)
    # fewer event pairs than launches: the rest are counted, not bracketed
    few = events(2)
    _, _, kb2, nb2 = vp.backward_traced(H, W, lab, lse, None, R, few)
    torch.cuda.synchronize()
    assert kb2 == ["other", "recompute"] and nb2 == nb
