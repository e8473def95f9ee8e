"""GPU parity of the owner-side Muon step: the HIP library (through the C ABI
binding) against the fp64 oracle on the same seeded inputs.

Bars: momentum buffer <= 1e-6 relative Frobenius; Newton-Schulz output
<= 2e-2 (bf16 chain) or <= 1e-4 (fp32 checking mode); parameters within one
bf16 ulp plus the update's share of the O error, and mostly bit-equal to the
rounded oracle value.
"""

import numpy as np
import pytest

from _gpu_util import Case, check_step, rel_fro, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nsd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import newton_schulz_dmuon_amd as m
    m.load()
    return m


SHAPES = [
    (128, 256),     # one fp32-sized tile, wide
    (300, 700),     # 2 x 3 tiles, ragged both ways
    (700, 300),     # tall: transposed path
    (513, 513),     # square, one row/col past a tile boundary
    (17, 33),
    (1, 1),
    (1, 300),
    (300, 1),
    (256, 256),     # exactly one tile
    (257, 1000),
    (1000, 257),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_single_matrix_bf16(nsd, shape):
    say(f"bf16 step {shape}")
    case = Case([shape], "bf16", "bf16", seed=1, m_std=1e-3)
    opts = nsd.StepOptions()
    err = check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))
    say(f"  O rel err {err:.3e}")


@pytest.mark.parametrize("shape", [(128, 256), (300, 700), (700, 300), (513, 513), (17, 33),
                                   (1, 300)])
def test_single_matrix_fp32_mode(nsd, shape):
    say(f"fp32-mode step {shape}")
    case = Case([shape], "f32", "f32", seed=2, g_std=1.0, m_std=0.5)
    opts = nsd.StepOptions(ns_fp32=True)
    err = check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))
    say(f"  O rel err {err:.3e}")


def test_tiny_fp32_workload(nsd):
    """One fp32 128x256 matrix, grad N(0,1), param N(0,0.02), zero momentum,
    mu 0.95, lr 0.02, 5 quintic steps; bf16 chain and fp32 mode."""
    from synth import matrix_inputs, workload
    w = workload(1)
    P, G, M = matrix_inputs(w, 0)
    for fp32 in (False, True):
        case = Case([(128, 256)], "f32", "f32")
        case.P, case.G, case.M = [P], [G], [M]
        opts = nsd.StepOptions(ns_fp32=fp32)
        err = check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))
        say(f"tiny workload fp32={fp32}: O rel err {err:.3e}")


@pytest.mark.parametrize("k", [0, 1, 2, 3, 8])
def test_ns_steps(nsd, k):
    case = Case([(300, 700), (700, 300)], "bf16", "bf16", seed=3, m_std=1e-3)
    opts = nsd.StepOptions(ns_steps=k)
    check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))


@pytest.mark.parametrize("fp32", [False, True])
def test_nesterov(nsd, fp32):
    dt = "f32" if fp32 else "bf16"
    case = Case([(300, 700), (513, 260)], dt, dt, seed=4, m_std=1e-3)
    opts = nsd.StepOptions(nesterov=True, ns_fp32=fp32)
    check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))


def test_mixed_dtypes_and_coefficients(nsd):
    case = Case([(200, 330)], "f32", "bf16", seed=5, m_std=1e-3)
    opts = nsd.StepOptions(a=1.5, b=-0.5, c=0.0, ns_steps=7, lr=0.1, momentum=0.9)
    check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))
    case = Case([(330, 200)], "bf16", "f32", seed=6, g_std=1.0)
    opts = nsd.StepOptions(a=2.0, b=-1.3, c=0.4, ns_steps=4)
    check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))


@pytest.mark.parametrize("c", [1e-30, 1e-40, 0.0])
def test_square_term_with_tiny_c(nsd, c):
    """The Square stage takes its b*A term from the operand tiles as (b/c)*A
    when b/c is finite (1e-30) and reads A instead when it is not (1e-40:
    b/c overflows fp32) or c = 0: all three agree with the oracle."""
    case = Case([(300, 700), (513, 513)], "bf16", "bf16", seed=9, m_std=1e-3)
    opts = nsd.StepOptions(a=1.5, b=-0.5, c=c, ns_steps=7, lr=0.1, momentum=0.9)
    err = check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))
    say(f"  c={c}: O rel err {err:.3e}")


def test_heterogeneous_group(nsd):
    """Many shapes in one grouped launch per stage."""
    shapes = [(300, 700), (700, 300), (17, 33), (513, 513), (1, 1), (256, 1024), (1024, 256),
              (64, 64), (129, 900)]
    case = Case(shapes, "bf16", "bf16", seed=7, m_std=1e-3)
    opts = nsd.StepOptions()
    check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))


def test_zero_gradient_and_momentum(nsd):
    case = Case([(300, 700)], "bf16", "bf16", seed=8)
    case.G = [np.zeros_like(case.G[0])]
    opts = nsd.StepOptions()
    P, M, O = case.run_gpu(opts)
    assert np.all(O[0] == 0) and np.all(M[0] == 0)
    assert np.array_equal(P[0], case.P[0].astype(np.float64))


def test_nonfinite_input_propagates_within_its_matrix(nsd):
    """Non-finite inputs propagate and are not clamped (reading R13): a NaN in
    one gradient element makes that momentum element NaN, the matrix's norm
    NaN and so its whole O and P; the other matrix of the same grouped
    launches is unaffected and matches the oracle."""
    case = Case([(300, 700), (257, 1000)], "bf16", "bf16", seed=21, m_std=1e-3)
    g0 = case.G[0].copy()
    g0[5, 7] = np.nan
    case.G[0] = g0
    opts = nsd.StepOptions()
    P, M, O = case.run_gpu(opts)
    nan_m = np.isnan(M[0])
    assert nan_m[5, 7] and nan_m.sum() == 1
    assert np.all(np.isnan(O[0])) and np.all(np.isnan(P[0]))
    clean = Case([(257, 1000)], "bf16", "bf16")
    clean.P, clean.G, clean.M, clean.scales = case.P[1:], case.G[1:], case.M[1:], case.scales[1:]
    err = check_step(clean, opts, (P[1:], M[1:], O[1:]), clean.run_oracle(opts))
    say(f"  clean matrix O rel err {err:.3e}")


@pytest.mark.parametrize("gram_ns", [False, True])
def test_qwen25_1p5b_layer(nsd, gram_ns):
    """One Qwen2.5-1.5B layer's projections: q/o 1536^2, k/v 256x1536,
    gate/up 8960x1536, down 1536x8960, bf16; the direct chain for every
    matrix, and the Gram-space chain (k, v, gate, up, down take it, q and o
    keep the direct one), as bench.py runs this workload."""
    from synth import matrix_inputs, workload
    w = workload(2)
    case = Case([(r, c) for _, r, c in w.shapes], "bf16", "bf16")
    case.P, case.G, case.M = [], [], []
    for i in range(len(w.shapes)):
        P, G, M = matrix_inputs(w, i)
        case.P.append(P); case.G.append(G); case.M.append(M)
    opts = nsd.StepOptions(gram_ns=gram_ns)
    say(f"qwen layer: gpu, gram_ns {gram_ns}")
    gpu = case.run_gpu(opts)
    say("qwen layer: oracle")
    err = check_step(case, opts, gpu, case.run_oracle(opts))
    say(f"  worst O rel err {err:.3e}")


def test_deterministic(nsd):
    case = Case([(300, 700), (700, 300), (513, 513)], "bf16", "bf16", seed=9, m_std=1e-3)
    opts = nsd.StepOptions()
    a = case.run_gpu(opts)
    b = case.run_gpu(opts)
    for x, y in zip(a, b):
        for u, v in zip(x, y):
            assert np.array_equal(u, v)


def test_workspace_reuse_across_shapes(nsd):
    """A workspace sized for a large call, reused by a smaller one."""
    ws = nsd.Workspace()
    for shapes in ([(700, 900)], [(300, 200), (17, 33)]):
        case = Case(shapes, "bf16", "bf16", seed=10, m_std=1e-3)
        opts = nsd.StepOptions()
        check_step(case, opts, case.run_gpu(opts, workspace=ws), case.run_oracle(opts))


def test_grads_read_from_packed_buffer(nsd):
    """Descriptors whose grad pointers point into one packed gradient buffer."""
    from oracle import partition as refp
    shapes = [(300, 700), (17, 33), (700, 300)]
    case = Case(shapes, "bf16", "bf16", seed=11)
    offs, total = refp.pack_offsets([r * c for r, c in shapes], 128)
    packed = torch.zeros(total, dtype=torch.bfloat16, device="cuda")
    G = []
    for g, o in zip(case.G, offs):
        view = packed[o:o + g.size].view(g.shape)
        view.copy_(to_dev(g, "bf16"))
        G.append(view)
    P = [to_dev(p, "bf16") for p in case.P]
    M = [to_dev(m, "f32") for m in case.M]
    O = [torch.empty_like(p) for p in P]
    opts = nsd.StepOptions()
    nsd.muon_step(P, G, M, case.scales, opts, orth_out=O)
    torch.cuda.synchronize()
    check_step(case, opts, ([to_host(p) for p in P], [to_host(m) for m in M],
                            [to_host(o) for o in O]), case.run_oracle(opts))


@pytest.mark.parametrize("gram", [False, True])
def test_check_finite_flags(nsd, gram):
    """DMUON_FLAG_CHECK_FINITE reports, per matrix, a NaN or an Inf in U: a
    NaN gradient element, an Inf momentum element, and a clean matrix.  The
    flags are rewritten by every step (a clean second step reads 0), and the
    outputs are those of a step without the flag, bit for bit."""
    shapes = [(300, 700), (257, 1000), (700, 300)]
    case = Case(shapes, "bf16", "bf16", seed=22, m_std=1e-3)
    g0 = case.G[0].copy()
    g0[3, 5] = np.nan
    m1 = case.M[1].copy()
    m1[7, 9] = np.inf
    ws = nsd.Workspace()
    opts = nsd.StepOptions(check_finite=True, gram_ns=gram)
    plain = nsd.StepOptions(gram_ns=gram)
    outs = {}
    for name, o in (("checked", opts), ("plain", plain)):
        bad = Case(shapes, "bf16", "bf16", seed=22, m_std=1e-3)
        bad.G[0], bad.M[1] = g0, m1
        outs[name] = bad.run_gpu(o, workspace=ws)
        if name == "checked":
            flags = nsd.nonfinite_flags([to_dev(p, "bf16") for p in bad.P], opts, ws).cpu().tolist()
    say(f"  flags {flags}")
    assert flags == [1, 1, 0]
    for x, y in zip(outs["checked"], outs["plain"]):
        for u, v in zip(x, y):
            assert np.array_equal(u, v, equal_nan=True)
    clean = Case(shapes, "bf16", "bf16", seed=23, m_std=1e-3)
    clean.run_gpu(opts, workspace=ws)
    flags = nsd.nonfinite_flags([to_dev(p, "bf16") for p in clean.P], opts, ws).cpu().tolist()
    assert flags == [0, 0, 0]


def test_side_stream_with_temporary_workspace(nsd):
    """A step enqueued on a side stream with no persisted workspace: the
    binding's temporary workspace is freed when the call returns, while the
    step's kernels still run on the side stream.  A buffer of the same size
    allocated on the current stream right after, and filled there, must not
    receive that memory (the binding marks it as in use by the side
    stream); the step's results match the oracle."""
    shapes = [(1024, 3072), (2048, 1024)]
    case = Case(shapes, "bf16", "bf16", seed=12, m_std=1e-3)
    opts = nsd.StepOptions(gram_ns=True)
    P = [to_dev(p, "bf16") for p in case.P]
    G = [to_dev(g, "bf16") for g in case.G]
    M = [to_dev(m, "f32") for m in case.M]
    O = [torch.empty_like(p) for p in P]
    need = nsd.workspace_bytes(P, opts)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    say(f"side-stream step, workspace {need} bytes")
    nsd.muon_step(P, G, M, case.scales, opts, orth_out=O, stream=side)
    junk = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    junk.fill_(0xFF)
    torch.cuda.synchronize()
    gpu = ([to_host(p) for p in P], [to_host(m) for m in M], [to_host(o) for o in O])
    err = check_step(case, opts, gpu, case.run_oracle(opts))
    say(f"  O rel err {err:.3e}")


SMALL = [(1, 300), (300, 1), (8, 50), (17, 33), (17, 100), (32, 200), (200, 32), (64, 400),
         (100, 100), (127, 500)]


@pytest.mark.parametrize("k", [5, 8])
def test_small_matrices_run_in_fp32(nsd, k):
    """In a bf16 step, matrices with min(r, c) < 128 run their chain in fp32
    (their singular values sit in the quintic's band for most iterations,
    where bf16 storage reaches about 2e-2 at five iterations and 3e-2 at
    eight): O within 1e-4 of fp64, plus the rounding of orth_out to bf16;
    a 128-wide matrix of the same call keeps the bf16 chain."""
    from _gpu_util import TOL_O_FP32
    shapes = SMALL + [(128, 512)]
    kinds = [kd for kd, f in nsd.step_launches(shapes, nsd.StepOptions(ns_steps=k)) if f > 0]
    assert kinds.count("final") == 2
    say(f"small matrices, ns_steps {k}")
    case = Case(SMALL, "bf16", "bf16", seed=60 + k, m_std=1e-3)
    opts = nsd.StepOptions(ns_steps=k, gram_ns=True)
    err = check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts), tol_o=TOL_O_FP32)
    say(f"  worst O rel err {err:.3e}")


@pytest.mark.parametrize("shapes,k,gram,fp32", [
    ([(2048, 2048)], 5, False, False),      # Gram splits (36 tiles of 32 steps)
    ([(2048, 2048)], 8, False, False),      # with B's pairs: Apply and Final split too
    ([(2048, 4608)], 6, True, False),       # Gram-space chain, P and T pairs
    ([(2048, 2048)], 5, False, True),       # fp32 mode: 64-step tiles, every stage split
    ([(2048, 2048), (300, 700)], 5, True, False),   # tiles of one and of several pieces side by side
])
def test_split_k_stages(nsd, shapes, k, gram, fp32):
    """Launches with fewer tiles than CUs run as pieces over K plus a reduce
    launch (the plan shows each split stage as a piece launch and a reduce
    launch of the same kind); the result matches the oracle."""
    opts = nsd.StepOptions(ns_steps=k, gram_ns=gram, ns_fp32=fp32)
    L = nsd.step_launches(shapes, opts)
    assert any(f == 0 for kd, f in L if kd in ("gram", "square", "apply", "final"))
    dt = "f32" if fp32 else "bf16"
    case = Case(shapes, dt, dt, seed=70 + k, m_std=1e-3)
    say(f"split-K step {shapes}, ns_steps {k}, gram_ns {gram}, fp32 {fp32}")
    err = check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))
    say(f"  worst O rel err {err:.3e}")


@pytest.mark.parametrize("shapes,k,gram", [
    ([(1000, 1500)], 5, False),                          # 8 x 8 128-tiles, the last rows ragged
    ([(1000, 1500), (129, 640)], 8, False),              # B's pairs; 2 x 2 beside 8 x 8
    ([(1536, 1536), (256, 1536), (1536, 4608)], 6, True),  # Gram-space chain beside the direct one
    ([(1536, 1536), (256, 1536), (1536, 8960)], 5, True),  # Qwen2.5-1.5B shapes: q, k, down
])
def test_square_launches_of_128_tiles(nsd, shapes, k, gram):
    """Square launches with fewer 256-tiles than CUs run 128 x 128 tiles
    (two work-groups per CU; diagonal tiles skip their below-diagonal
    quarter and mirror the rest); the result matches the oracle."""
    opts = nsd.StepOptions(ns_steps=k, gram_ns=gram)
    L = nsd.step_launches(shapes, opts, tiles=True)
    assert any(kd == "square" and t == 128 for kd, _, t in L), L
    case = Case(shapes, "bf16", "bf16", seed=80 + k, m_std=1e-3)
    say(f"128-tile Square launches {shapes}, ns_steps {k}, gram_ns {gram}")
    err = check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))
    say(f"  worst O rel err {err:.3e}")


@pytest.mark.parametrize("shape", [(2, 1 << 22), (1 << 22, 3)])
def test_longest_side(nsd, shape):
    """A matrix at the step's limit of 2^22 elements per side (16-bit tile
    indices up to 16383, 32-bit row-block offsets): m < 128, so its chain
    runs in fp32; its one Gram tile has 131072 K steps and runs split over
    K, its Apply has 16384 tiles."""
    say(f"longest side {shape}")
    case = Case([shape], "bf16", "bf16", seed=13, m_std=1e-3)
    opts = nsd.StepOptions()
    err = check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))
    say(f"  O rel err {err:.3e}")
