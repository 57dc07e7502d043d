"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/vpce.h declares, sizes its workspace independently of
V, and rejects bad arguments before anything is enqueued (these calls make no
HIP call at all)."""
import ctypes
import os
import re

import pytest

import vocabulary_projection_cross_amd as vp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vpce.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vpce_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vp.library_path()):
        pytest.fail("libvpce.so is not built (run __graft_entry__.build())")
    return vp._load()


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert names == ["vpce_backward", "vpce_backward_traced", "vpce_forward",
                     "vpce_forward_noalloc", "vpce_forward_noalloc_bytes",
                     "vpce_forward_traced", "vpce_plan",
                     "vpce_ring_mode", "vpce_shard_backward",
                     "vpce_shard_fold", "vpce_state_finish",
                     "vpce_state_init", "vpce_status_string",
                     "vpce_workspace_bytes", "vpce_workspace_bytes_chunk"]
    for n in names:
        assert hasattr(lib, n), n
    out = os.popen(f"nm -D --defined-only {vp.library_path()}").read()
    exported = set(re.findall(r" T (vpce_\w+)", out))
    assert exported == set(names)


def test_status_strings(lib):
    for s in range(7):
        assert lib.vpce_status_string(s)
    assert lib.vpce_status_string(99) == b"unknown status"


@pytest.mark.parametrize("N,d,R", [(65536, 7168, 8), (131072, 5120, 7),
                                   (4096, 2048, 4), (1, 8, 1)])
def test_workspace_independent_of_v(lib, N, d, R):
    sizes = {lib.vpce_workspace_bytes(N, d, V, R, 0)
             for V in (R, 32000, 129280, 151936, 1 << 30)}
    assert len(sizes) == 1 and sizes.pop() > 0


def test_workspace_rejects_bad_shapes(lib):
    assert lib.vpce_workspace_bytes(10, 12, 100, 1, 0) == 0   # d % 8
    assert lib.vpce_workspace_bytes(10, 12, 100, 1, 1) > 0    # f32: d % 4
    assert lib.vpce_workspace_bytes(10, 16, 5, 6, 0) == 0     # R > V
    assert lib.vpce_workspace_bytes(-1, 16, 5, 1, 0) == 0
    assert lib.vpce_workspace_bytes(10, 16, 5, 1, 7) == 0     # dtype
    assert lib.vpce_workspace_bytes(10, 16, 1 << 31, 1, 0) == 0
    assert lib.vpce_workspace_bytes(0, 16, 5, 1, 0) > 0       # empty batch
    # hidden size: 320 rows of an fp32 operand must stay below 2^31 bytes
    assert lib.vpce_workspace_bytes(1, 1_000_000, 5, 1, 1) > 0
    assert lib.vpce_workspace_bytes(1, 1_000_008, 5, 1, 0) == 0
    assert lib.vpce_workspace_bytes(2_000_000, 16, 5, 1, 0) > 0
    assert lib.vpce_workspace_bytes(2_000_001, 16, 5, 1, 0) == 0


def _fwd(lib, H=8, W=16, lab=8, N=4, d=16, V=10, R=2, dt=0, loss=4, lse=4,
         ws=256, wsb=1 << 20):
    return lib.vpce_forward(H, W, lab, N, d, V, R, -100, dt, loss, lse, ws,
                            wsb, None)


def test_argument_errors_before_launch(lib):
    A = 1 << 20   # aligned fake addresses: never dereferenced on error paths
    assert _fwd(lib, H=A, W=A, lab=A, loss=A, lse=A, ws=A, dt=5) == 3
    assert _fwd(lib, H=A, W=A, lab=A, loss=A, lse=A, ws=A, R=11) == 2
    assert _fwd(lib, H=A, W=A, lab=A, loss=A, lse=A, ws=A, d=12) == 2
    assert _fwd(lib, H=None, W=A, lab=A, loss=A, lse=A, ws=A) == 1
    assert _fwd(lib, H=A, W=A, lab=A, loss=A, lse=A, ws=None) == 1
    assert _fwd(lib, H=A + 8, W=A, lab=A, loss=A, lse=A, ws=A) == 4
    assert _fwd(lib, H=A, W=A, lab=A, loss=A, lse=A, ws=A + 16) == 4
    assert _fwd(lib, H=A, W=A, lab=A, loss=A, lse=A, ws=A, wsb=16) == 5
    st = lib.vpce_backward(A, A, A, A, None, 4, 16, 10, 2, -100, 0, None, A,
                           A, 1 << 20, None)
    assert st == 1      # dH missing
    st = lib.vpce_backward(A, A, A, A, None, 4, 16, 10, 2, -100, 0, A, A, A,
                           16, None)
    assert st == 5
    # dH and dW take 16-byte vector stores: 4-byte alignment is not enough
    st = lib.vpce_backward(A, A, A, A, None, 4, 16, 10, 2, -100, 0, A + 4, A,
                           A, 1 << 20, None)
    assert st == 4
    st = lib.vpce_backward(A, A, A, A, None, 4, 16, 10, 2, -100, 0, A, A + 8,
                           A, 1 << 20, None)
    assert st == 4


def test_device_code_hash_reads_the_built_library():
    """bench.py keys stored counter readings on the library's device code."""
    import bench
    h = bench.kernel_code_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.kernel_code_hash() == h


def test_autograd_wrapper_has_no_host_path():
    """The differentiable wrapper rejects host tensors instead of computing
    anything on the CPU."""
    import torch
    import vocabulary_projection_cross_amd as vp
    from vocabulary_projection_cross_amd.autograd import cross_entropy
    H = torch.zeros((4, 16), dtype=torch.bfloat16, requires_grad=True)
    W = torch.zeros((10, 16), dtype=torch.bfloat16, requires_grad=True)
    lab = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(vp.VPCEError):
        cross_entropy(H, W, lab, 2)


def _caller_bytes(N, d, V, esz):
    """H, W, labels, lse, loss, dH, dW at their exact sizes."""
    return N * d * esz + V * d * esz + 8 * N + 4 * N + 4 + 4 * N * d + 4 * V * d


@pytest.mark.parametrize("N,d,V,R", [(65536, 7168, 129280, 8),
                                     (4096, 2048, 32000, 4), (300, 136, 1000, 3)])
def test_chunk_workspace_grows_with_the_chunk(lib, N, d, V, R):
    full = lib.vpce_workspace_bytes(N, d, V, R, 0)
    assert lib.vpce_workspace_bytes_chunk(N, d, V, R, 0, 8192) == full
    sizes = [lib.vpce_workspace_bytes_chunk(N, d, V, R, 0, c)
             for c in range(256, 8193, 256)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    assert sizes[0] < sizes[-1]
    for bad in (0, 128, 255, 300, 8448, 16384, -256):
        assert lib.vpce_workspace_bytes_chunk(N, d, V, R, 0, bad) == 0


@pytest.mark.parametrize("N,d,V,R,dt", [(65536, 7168, 129280, 8, 0),
                                        (4096, 2048, 32000, 4, 0),
                                        (300, 136, 1000, 3, 1)])
def test_planner_picks_the_widest_chunk_that_fits(N, d, V, R, dt):
    import torch
    dtype = torch.bfloat16 if dt == 0 else torch.float32
    esz = 2 if dt == 0 else 4
    fixed = _caller_bytes(N, d, V, esz)
    for C in (256, 4096, 6400, 8192):
        ws = vp.workspace_bytes(N, d, V, R, dtype, chunk_cols=C)
        exact = vp.plan(N, d, V, R, fixed + ws, dtype)
        assert exact == {"chunk_cols": C, "workspace_bytes": ws,
                         "peak_bytes": fixed + ws}
        if C > 256:
            below = vp.plan(N, d, V, R, fixed + ws - 1, dtype)
            assert below["chunk_cols"] < C
            assert below["peak_bytes"] <= fixed + ws - 1
    roomy = vp.plan(N, d, V, R, 1 << 50, dtype)
    assert roomy["chunk_cols"] == 8192
    assert roomy["workspace_bytes"] == vp.workspace_bytes(N, d, V, R, dtype)
    ws256 = vp.workspace_bytes(N, d, V, R, dtype, chunk_cols=256)
    with pytest.raises(vp.VPCEError, match="status 5"):
        vp.plan(N, d, V, R, fixed + ws256 - 1, dtype)


def test_planner_argument_errors(lib):
    c, w, pk = ctypes.c_int64(-7), ctypes.c_size_t(3), ctypes.c_size_t(4)
    assert lib.vpce_plan(10, 12, 100, 1, 0, 1 << 40, ctypes.byref(c),
                         ctypes.byref(w), ctypes.byref(pk)) == 2   # d % 8
    assert lib.vpce_plan(10, 16, 100, 1, 0, 1 << 40, None, ctypes.byref(w),
                         ctypes.byref(pk)) == 1
    assert lib.vpce_plan(10, 16, 100, 1, 0, 100, ctypes.byref(c),
                         ctypes.byref(w), ctypes.byref(pk)) == 5
    assert (c.value, w.value, pk.value) == (-7, 3, 4)   # left untouched


def test_ring_mode_rule_on_the_workloads():
    """Weights move exactly when the widest shard has fewer rows than the
    batch has tokens; the payloads are N*d*b and ceil(V/R)*d*b."""
    import torch
    import workloads as WL
    modes = {}
    for w in WL.WORKLOADS:
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        esz = 2 if w.dtype == "bf16" else 4
        m = vp.ring_mode(w.N, w.d, w.V, w.R, dt)
        widest = -(-w.V // w.R)
        assert m["activation_bytes"] == w.N * w.d * esz
        assert m["weight_bytes"] == widest * w.d * esz
        modes[w.name] = m["mode"]
        assert m["mode"] == (vp.MOVE_WEIGHTS if widest < w.N
                             else vp.MOVE_ACTIVATIONS)
    # the 4096-token workload has 8000-row shards: its batches travel
    assert sorted(modes.values()).count(vp.MOVE_ACTIVATIONS) == 2
    assert vp.ring_mode(100, 8, 1000, 10)["mode"] == vp.MOVE_ACTIVATIONS
    assert vp.ring_mode(101, 8, 1000, 10)["mode"] == vp.MOVE_WEIGHTS


def test_shard_calls_reject_bad_arguments(lib):
    A = 1 << 20   # aligned fake addresses: never dereferenced on error paths
    fold = lambda **k: lib.vpce_shard_fold(
        k.get("H", A), k.get("W", A), A, 4, 16, 10, k.get("vb", 0),
        k.get("vc", 5), -100, 0, k.get("st", A), A, k.get("wsb", 1 << 20),
        None)
    assert fold(vb=6, vc=5) == 2          # past the vocabulary
    assert fold(vb=-1) == 2
    assert fold(vc=0) == 2
    assert fold(W=None) == 1
    assert fold(st=None) == 1
    assert fold(H=A + 8) == 4
    assert fold(wsb=16) == 5
    assert lib.vpce_state_init(None, 4, None) == 1
    assert lib.vpce_state_init(None, -1, None) == 2
    assert lib.vpce_state_init(None, 0, None) == 0   # nothing to do
    assert lib.vpce_state_finish(A, A, 4, -100, A, None, None, A, 1 << 20,
                                 None) == 1          # totals
    assert lib.vpce_state_finish(A, A, 4, -100, A, A + 4, None, A, 1 << 20,
                                 None) == 4          # totals fp64-aligned
    assert lib.vpce_state_finish(A, A, 4, -100, A, A, None, A, 8,
                                 None) == 5
    bwd = lambda **k: lib.vpce_shard_backward(
        A, A, A, A, k.get("tot", A), None, 4, 16, 10, k.get("vb", 2), 5,
        -100, 0, A, k.get("dW", A), A, k.get("wsb", 1 << 20), None)
    assert bwd(vb=6) == 2
    assert bwd(tot=None) == 1
    assert bwd(dW=None) == 1
    assert bwd(dW=A + 4) == 4
    assert bwd(wsb=64) == 5
    mode, act, wts = ctypes.c_int32(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.vpce_ring_mode(4, 12, 10, 1, 0, ctypes.byref(mode),
                              ctypes.byref(act), ctypes.byref(wts)) == 2
    assert lib.vpce_ring_mode(4, 16, 10, 2, 0, None, ctypes.byref(act),
                              ctypes.byref(wts)) == 1


def test_bench_traffic_record_goes_stale_with_the_device_code(tmp_path,
                                                             monkeypatch):
    """A stored counter reading is used only while the device code it was
    taken on is the one built now."""
    import json
    import bench
    built = bench.kernel_code_hash()
    rec = {"kernel_code_hash": built, "hbm_bytes_per_launch": 123}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "prod_kernel_traffic_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_code_hash", lambda: built)
    k = "prod_kernel (dH += G W)"
    assert bench.traffic_record("w", k)["hbm_bytes_per_launch"] == 123
    assert bench.traffic_record("w", "fwd_lse_kernel") is None
    rec["chunk_cols"] = 8192
    (prof / "prod_kernel_traffic_w.json").write_text(json.dumps(rec))
    assert bench.traffic_record("w", k, 8192)["hbm_bytes_per_launch"] == 123
    assert bench.traffic_record("w", k, 4096) is None
    rec["kernel_code_hash"] = "0" * 16
    (prof / "prod_kernel_traffic_w.json").write_text(json.dumps(rec))
    assert bench.traffic_record("w", k) is None
    assert bench.traffic_record("missing", k) is None


def test_bench_kernel_table_from_event_pairs():
    """Per-kernel figures of the bench line: launches per step, mean launch
    time over the timed steps, and flops per launch from the chunk widths
    (shards in ring order, each cut into chunks of at most C columns)."""
    import bench
    import workloads as WL

    class Ev:
        def __init__(self, t):
            self.t = t

        def elapsed_time(self, other):
            return other.t - self.t

    w = WL.custom(N=1000, d=64, V=10, R=3, name="t")   # shards 4, 3, 3
    assert bench.chunk_widths(w, 2) == [2, 2, 2, 1, 2, 1]
    assert bench.chunk_widths(w, 16384) == [4, 3, 3]
    kinds_f = ["other", "forward_tile", "merge", "other"]
    kinds_b = ["other"] + ["recompute", "products"] * 3

    def evs(kinds, steps, dur):
        out = []
        for s in range(steps):
            e = []
            for i, k in enumerate(kinds):
                e += [Ev(0.0), Ev(dur(k, i) * (1 + s))]
            out.append(e)
        return out

    fev = evs(kinds_f, 2, lambda k, i: 4.0 if k == "forward_tile" else 0.01)
    bev = evs(kinds_b, 2, lambda k, i: {"products": 3.0}.get(k, 0.5))
    t = bench.kernel_table(w, kinds_f, fev, kinds_b, bev, 16384)
    # durations of step s are (1 + s) x base: the mean over 2 steps is 1.5 x
    assert t["forward_tile"]["launches_per_step"] == 1
    assert t["forward_tile"]["launch_ms"] == 6.0
    assert t["forward_tile"]["flops_per_launch"] == 2.0 * 1000 * 64 * 10
    assert t["products"]["launches_per_step"] == 3
    assert t["products"]["ms_per_step"] == 13.5
    # both products of chunks of 4, 3 and 3 columns: 4 N d (10 / 3) per launch
    assert t["products"]["flops_per_launch"] == 4.0 * 1000 * 64 * 10 / 3
    assert t["recompute"]["flops_per_launch"] == 2.0 * 1000 * 64 * 10 / 3
    assert "frac" not in t["other"]
    assert t["other"]["launches_per_step"] == 3
    dom = max(t, key=lambda k: t[k]["ms_per_step"])
    assert dom == "products"


def test_bench_clock_sampler_without_the_tool(monkeypatch):
    """Without amd-smi (or when it fails) the sampled clock is reported as
    None instead of failing the benchmark."""
    import subprocess
    import bench

    def boom(*a, **k):
        raise FileNotFoundError("amd-smi")
    monkeypatch.setattr(subprocess, "run", boom)
    with bench.ClockSampler() as c:
        pass
    assert c.median() is None and c.samples == []


def test_bench_refuses_several_gpus():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("defines", [["-DVPCE_MFMA_BLOCK=32"],
                                     ["-DVPCE_RING_RB=64",
                                      "-DVPCE_RING_NST=4",
                                      "-DVPCE_WIDE_COLS=256"]])
def test_engine_build_options_compile(tmp_path, defines):
    """The engine's build options for the forward and the logit recompute
    (32 x 32 MFMA blocks; a deeper ring of 64-byte slabs on 256-column
    tiles) still compile for gfx950; the default build is what build() makes
    and the GPU tests run."""
    from vocabulary_projection_cross_amd import build as B
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc is not installed")
    src = os.path.join(B.CSRC, "vpce.hip")
    out = tmp_path / "vpce.o"
    import subprocess
    r = subprocess.run([B.HIPCC, *B.HIP_FLAGS, *defines, "-I", B.INCLUDE,
                        "-I", B.CSRC, "--cuda-device-only", "-c", src,
                        "-o", str(out)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]


def test_traced_calls_check_their_trace_arguments(lib):
    """The timed variants refuse bad trace arguments before anything is
    enqueued (no GPU is touched on these paths)."""
    import ctypes
    A = 1 << 20                       # any 256-aligned address; never read
    n = ctypes.c_int32(0)
    kinds = (ctypes.c_int32 * 4)()
    evs = (ctypes.c_void_p * 8)(*([A] * 8))

    def fwd(events, cap, k, used):
        return lib.vpce_forward_traced(A, A, A, 4, 16, 10, 2, -100, 0, A, A,
                                       A, 1 << 20, None, events, cap, k, used)

    def bwd(events, cap, k, used):
        return lib.vpce_backward_traced(A, A, A, A, None, 4, 16, 10, 2, -100,
                                        0, A, A, A, 1 << 20, None, events,
                                        cap, k, used)

    for call in (fwd, bwd):
        assert call(evs, -1, kinds, ctypes.byref(n)) == 2
        assert call(None, 4, kinds, ctypes.byref(n)) == 1
        assert call(evs, 4, None, ctypes.byref(n)) == 1
        assert call(evs, 4, kinds, None) == 1
        holes = (ctypes.c_void_p * 8)(*([A] * 7 + [None]))
        assert call(holes, 4, kinds, ctypes.byref(n)) == 1
        # argument errors of the untimed call come through unchanged
    assert lib.vpce_forward_traced(A, A, A, 4, 12, 10, 2, -100, 0, A, A, A,
                                   1 << 20, None, evs, 4, kinds,
                                   ctypes.byref(n)) == 2
    assert lib.vpce_backward_traced(A, A, A, A, None, 4, 16, 10, 2, -100, 0,
                                    A, A, A, 64, None, evs, 4, kinds,
                                    ctypes.byref(n)) == 5
