"""Host-side launch plan of the step (dmuon_step_launches), no GPU: which
matrices take the Gram-space chain, its phase split, the launch sequence
and the algorithmic flop count of every launch."""

import ctypes
import math

import pytest

nsd = pytest.importorskip("newton_schulz_dmuon_amd")
from newton_schulz_dmuon_amd import _lib  # noqa: E402

LLAMA8B_OWNER0 = [(4096, 4096)] * 8 + [(1024, 4096)] * 8 + [(14336, 4096)] * 8 + \
    [(4096, 14336)] * 4


def pairs(k, fp32=False):
    """From six iterations on, the bf16 chain stores B / P as hi + lo pairs."""
    return k >= 6 and not fp32


def small(m, fp32=False):
    """In a bf16 step, matrices with m < 128 run their chain in fp32 (no pairs)."""
    return m < 128 and not fp32


def direct_flops(m, n, k, fp32=False):
    """Executed flops: with pairs, Apply runs a second pass over B's low half
    from the third iteration on."""
    paired = max(k - 2, 0) if pairs(k, fp32) and not small(m, fp32) else 0
    return k * (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n) + paired * 2 * m * m * n


def uses_gram(m, n, k, gram):
    return gram and k >= 5 and n >= 2 * m and m >= 128


def phases(k):
    return [2] * (k // 2) + ([1] if k % 2 else [])


def square_passes(L, split):
    """Products of m_p x m_p matrices in a phase of L iterations, counted in
    full passes: L of P, L - 1 of P P, L - 1 of A T, L - 1 of Q P.  With
    pairs, P P reads a pair on both sides (3 passes), the first Q P too
    (Q is the first P), later ones on one side (2), and A T reads T's pair
    (2)."""
    if not split:
        return 4 * L - 3
    return L + 3 * (L - 1) + 2 * (L - 1) + (3 + 2 * (L - 2) if L >= 2 else 0)


def gram_flops(m, n, k, fp32=False):
    ph = phases(k)
    split = pairs(k, fp32)
    apply = sum(2 if split and L == 1 else 1 for L in ph) * 2 * m * m * n
    return len(ph) * m * (m + 1) * n + apply + \
        sum(square_passes(L, split) for L in ph) * m * m * (m + 1)


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7, 8, 10])
def test_phase_split(k):
    ph = phases(k)
    assert sum(ph) == k and max(ph) <= 2 and ph == sorted(ph, reverse=True)
    kinds = [kd for kd, _ in nsd.step_launches([(256, 1024)], nsd.StepOptions(ns_steps=k, gram_ns=True))]
    assert kinds[:2] == ["momentum_orient", "norm"] and kinds[-1] == "final"
    if k < 5:   # fewer than five iterations keep the direct chain
        assert kinds[2:] == ["gram", "square", "apply"] * (k - 1) + ["gram", "square", "final"]
        return
    assert kinds.count("gram") == len(ph)
    assert kinds.count("apply") == len(ph) - 1
    # per phase of L >= 2: L launches of P, L - 1 of A P^2, and L of P^2 and / or
    # Q P (one launch where both run); a phase of 1 is P alone
    assert kinds.count("square") == sum(3 * L - 1 if L > 1 else 1 for L in ph)


def test_direct_chain_sequence_and_flops():
    L = nsd.step_launches(LLAMA8B_OWNER0, nsd.StepOptions())
    kinds = [k for k, _ in L]
    assert kinds == ["momentum_orient", "norm"] + ["gram", "square", "apply"] * 4 + \
        ["gram", "square", "final"]
    total = sum(f for _, f in L)
    want = sum(direct_flops(min(r, c), max(r, c), 5) for r, c in LLAMA8B_OWNER0)
    assert total == want
    assert abs(total - 58.98e12) < 0.01e12


def test_gram_chain_selection_and_flops():
    shapes = LLAMA8B_OWNER0 + [(300, 599), (300, 600), (601, 300), (128, 256), (127, 256)]
    L = nsd.step_launches(shapes, nsd.StepOptions(gram_ns=True))
    total = sum(f for _, f in L)
    want = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        want += gram_flops(m, n, 5) if uses_gram(m, n, 5, True) else direct_flops(m, n, 5)
    assert total == want
    # the two bf16 chains' launches of the same kind share grouped launches:
    # one final for them, one for the small matrix's fp32 chain (127 x 256),
    # and fewer launches than the two chains run apart
    kinds = [k for k, _ in L]
    assert kinds.count("final") == 2
    assert kinds[-15:] == ["gram", "square", "apply"] * 4 + ["gram", "square", "final"]
    shapes = shapes[:-1]
    L = nsd.step_launches(shapes, nsd.StepOptions(gram_ns=True))
    kinds = [k for k, _ in L]
    assert kinds.count("final") == 1
    alone = len(nsd.step_launches(shapes[:8], nsd.StepOptions(gram_ns=True))) + \
        len(nsd.step_launches(shapes[8:28], nsd.StepOptions(gram_ns=True))) - 2
    assert len(L) < alone


def test_gram_needs_more_workspace():
    def ws(opts, shapes):
        arr = (_lib.Matrix * len(shapes))()
        for i, (r, c) in enumerate(shapes):
            arr[i] = _lib.Matrix(None, 0, 0, None, None, None, r, c, 1.0, 0, 0)
        out = ctypes.c_size_t(0)
        cfg = opts.to_c()
        _lib.check(_lib.load().dmuon_workspace_bytes(arr, len(shapes), ctypes.byref(cfg),
                                                     ctypes.byref(out)))
        return out.value
    for shapes, extra in (([(300, 700)], 4 * 512 * 512 * 2), ([(300, 500)], 0),
                          ([(513, 513)], 0)):
        # four more m_p x m_p buffers per Gram-space matrix, plus its launch tables
        d = ws(nsd.StepOptions(gram_ns=True), shapes) - ws(nsd.StepOptions(), shapes)
        assert extra <= d < extra + 65536 and (d == 0) == (extra == 0), (shapes, d)


def test_pairs_add_workspace_not_launches():
    """From six iterations on: one more m_p x m_p buffer per direct-chain
    matrix (B's low half) and three per Gram-space matrix (the low halves of
    the first and the later P and of T); the launch sequence is the same,
    and the fp32 mode has no pairs."""
    def ws(opts, shapes):
        arr = (_lib.Matrix * len(shapes))()
        for i, (r, c) in enumerate(shapes):
            arr[i] = _lib.Matrix(None, 0, 0, None, None, None, r, c, 1.0, 0, 0)
        out = ctypes.c_size_t(0)
        cfg = opts.to_c()
        _lib.check(_lib.load().dmuon_workspace_bytes(arr, len(shapes), ctypes.byref(cfg),
                                                     ctypes.byref(out)))
        return out.value
    buf = 512 * 512 * 2
    for gram, shapes, extra in ((False, [(300, 700)], buf), (True, [(300, 700)], 3 * buf),
                                (True, [(700, 300)], 3 * buf), (True, [(513, 300)], buf),
                                (True, [(100, 700)], 0)):
        o5 = nsd.StepOptions(ns_steps=5, gram_ns=gram)
        o6 = nsd.StepOptions(ns_steps=6, gram_ns=gram)
        k5 = [kd for kd, _ in nsd.step_launches(shapes, o5)]
        k6 = [kd for kd, _ in nsd.step_launches(shapes, o6)]
        d = ws(o6, shapes) - ws(o5, shapes)
        assert extra <= d < extra + 65536, (gram, shapes, d)
        if not gram or shapes in ([(513, 300)], [(100, 700)]):   # the direct chain: one more iteration
            assert k6 == k5[:2] + ["gram", "square", "apply"] + k5[2:]
        f6 = nsd.StepOptions(ns_steps=6, gram_ns=gram, ns_fp32=True)
        f5 = nsd.StepOptions(ns_steps=5, gram_ns=gram, ns_fp32=True)
        assert ws(f6, shapes) == ws(f5, shapes)


def test_step_launches_errors():
    lib = _lib.load()
    arr = (_lib.Matrix * 1)(_lib.Matrix(None, 0, 0, None, None, None, 8, 8, 1.0, 0, 0))
    cfg = nsd.StepOptions().to_c()
    cnt = ctypes.c_int32(0)
    assert lib.dmuon_step_launches(arr, 1, ctypes.byref(cfg), None, 0, None) == _lib.ERR_INVALID_ARG
    assert lib.dmuon_step_launches(arr, 1, ctypes.byref(cfg), None, 2, ctypes.byref(cnt)) == \
        _lib.ERR_INVALID_ARG
    assert lib.dmuon_step_launches(arr, 1, ctypes.byref(cfg), None, 0, ctypes.byref(cnt)) == _lib.OK
    assert cnt.value == 17
    bad = _lib.Matrix(None, 0, 0, None, None, None, 0, 8, 1.0, 0, 0)
    arr2 = (_lib.Matrix * 1)(bad)
    assert lib.dmuon_step_launches(arr2, 1, ctypes.byref(cfg), None, 0, ctypes.byref(cnt)) == \
        _lib.ERR_INVALID_ARG
    out = (_lib.LaunchInfo * 4)()
    assert lib.dmuon_step_launches(arr, 1, ctypes.byref(cfg), out, 4, ctypes.byref(cnt)) == _lib.OK
    assert cnt.value == 17 and [out[j].kind for j in range(4)] == [1, 2, 4, 5]
    # element-wise launches report no tile; an 8 x 8 matrix runs its chain
    # in fp32 on 256-tiles
    assert [out[j].tile for j in range(4)] == [0, 0, 256, 256]


@pytest.mark.parametrize("seed", range(12))
def test_random_plans_are_consistent(seed):
    """Random mixes of square, wide, tall and tiny matrices at every ns_steps
    up to 10, both chains: the library's own checks of the plan pass (every
    tile inside its launch's table and matrix; every output tile computed
    exactly once per launch, split tiles' pieces covering their K steps) and
    the flop count is the sum of the two chains' counts."""
    import numpy as np
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 30))
    shapes = []
    for _ in range(n):
        r = int(rng.choice([1, 17, 256, 300, 513, 1024, 2000]))
        c = int(rng.choice([1, 33, 256, 700, 1000, 4096]))
        shapes.append((r, c) if rng.random() < 0.5 else (c, r))
    for k in range(0, 11):
        for gram in (False, True):
            L = nsd.step_launches(shapes, nsd.StepOptions(ns_steps=k, gram_ns=gram))
            want = 0
            for r, c in shapes:
                m, nn = min(r, c), max(r, c)
                want += gram_flops(m, nn, k) if uses_gram(m, nn, k, gram) else direct_flops(m, nn, k)
            assert sum(f for _, f in L) == want
            if k > 0:
                n_small = any(small(min(r, c)) for r, c in shapes)
                n_big = any(not small(min(r, c)) for r, c in shapes)
                assert [x for x, f in L if f > 0].count("final") == n_small + n_big
                check_split_launches(L)


def check_split_launches(L):
    """A split stage is a launch of pieces (the stage's flops) followed by a
    launch of reduce entries of the same kind (no flops)."""
    gemm = ("gram", "square", "apply", "final", "gram_square")
    for j, (kind, f) in enumerate(L):
        if kind in gemm and f == 0:
            assert j > 0 and L[j - 1][0] == kind and L[j - 1][1] > 0, (j, L)


def test_split_k_where_launches_leave_cus_idle():
    """Qwen2.5-1.5B layer: its Gram launches (about a hundred tiles, up to
    140 K steps) run split; the Llama-3.1-8B share (1088+ tiles per launch)
    and short-K launches (24 steps) do not.  A single 2048 x 2048 matrix
    splits its symmetric stages, and Apply too where its K loop is long."""
    from synth import workload
    w = workload(2)
    shapes = [(r, c) for _, r, c in w.shapes]
    for gram in (False, True):
        L = nsd.step_launches(shapes, nsd.StepOptions(gram_ns=gram))
        check_split_launches(L)
        reduces = [k for k, f in L if k in ("gram", "square", "apply", "final") and f == 0]
        assert reduces and set(reduces) == {"gram"}, reduces
    L = nsd.step_launches(LLAMA8B_OWNER0, nsd.StepOptions(gram_ns=True))
    assert all(f > 0 for k, f in L if k in ("gram", "square", "apply", "final"))
    # a single 2048 x 2048 matrix: 36 symmetric Gram tiles of 32 K steps
    # split (its Square launches run 128-tiles instead); 64 Apply tiles of 32
    # steps do not (two pieces would not pay for the reduce), but do when B's
    # pairs double Apply's K loop (ns_steps 8); in the fp32 mode (64 steps of
    # 32 elements, no 128-tiles) every stage splits
    def split_kinds(opts):
        L = nsd.step_launches([(2048, 2048)], opts)
        check_split_launches(L)
        assert sum(f for _, f in L) == direct_flops(2048, 2048, opts.ns_steps, opts.ns_fp32)
        return {k for k, f in L if k in ("gram", "square", "apply", "final") and f == 0}
    assert split_kinds(nsd.StepOptions()) == {"gram"}
    assert split_kinds(nsd.StepOptions(ns_steps=8)) == {"gram", "apply", "final"}
    assert split_kinds(nsd.StepOptions(ns_fp32=True)) == {"gram", "square", "apply", "final"}


def test_square_launches_with_few_tiles_run_128_tiles():
    """A bf16 Square launch whose 256-tiles would leave CUs idle runs
    128 x 128 tiles (four times the tiles, two work-groups per CU), never
    split; every other GEMM launch runs 256-tiles.  The Qwen2.5-1.5B layer's
    Square launches (78 upper-triangle 256-tiles at 1536) take 128-tiles; the
    Llama-3.1-8B share's (1088+ tiles per launch) do not, nor does the fp32
    mode."""
    from synth import workload
    w = workload(2)
    qwen = [(r, c) for _, r, c in w.shapes]
    for shapes, opts, want in ((qwen, nsd.StepOptions(), 128), (qwen, nsd.StepOptions(gram_ns=True), 128),
                               (qwen, nsd.StepOptions(ns_steps=8), 128),
                               (qwen, nsd.StepOptions(ns_fp32=True), 256),
                               (LLAMA8B_OWNER0, nsd.StepOptions(gram_ns=True), 256),
                               (LLAMA8B_OWNER0, nsd.StepOptions(), 256)):
        L = nsd.step_launches(shapes, opts, tiles=True)
        assert [(k, f) for k, f, _ in L] == nsd.step_launches(shapes, opts)
        for j, (k, f, t) in enumerate(L):
            if k in ("momentum_sumsq", "momentum_orient", "norm", "update_direct"):
                assert t == 0
            elif k == "square" and f > 0:
                assert t == want, (j, L)
                if t == 128:  # whole tiles: no reduce launch follows
                    assert j + 1 == len(L) or L[j + 1][:2] != ("square", 0.0)
            else:
                assert t == 256, (j, L)


def test_nonfinite_flags_offset():
    """DMUON_FLAG_CHECK_FINITE: the int32[n] flags sit 256-byte aligned inside
    the workspace, which grows by their slot; without the flag the offset
    call is an error."""
    lib = _lib.load()
    shapes = [(300, 700), (17, 33), (513, 513)]
    arr = (_lib.Matrix * 3)(*[_lib.Matrix(None, 0, 0, None, None, None, r, c, 1.0, 0, 0)
                              for r, c in shapes])
    off = ctypes.c_size_t(0)
    plain = nsd.StepOptions().to_c()
    assert lib.dmuon_nonfinite_flags_offset(arr, 3, ctypes.byref(plain), ctypes.byref(off)) == \
        _lib.ERR_INVALID_ARG
    for gram in (False, True):
        for k in (0, 5):
            opts = nsd.StepOptions(check_finite=True, gram_ns=gram, ns_steps=k)
            cfg = opts.to_c()
            assert lib.dmuon_nonfinite_flags_offset(arr, 3, ctypes.byref(cfg), None) == \
                _lib.ERR_INVALID_ARG
            assert lib.dmuon_nonfinite_flags_offset(arr, 3, ctypes.byref(cfg), ctypes.byref(off)) == \
                _lib.OK
            total, base = ctypes.c_size_t(0), ctypes.c_size_t(0)
            _lib.check(lib.dmuon_workspace_bytes(arr, 3, ctypes.byref(cfg), ctypes.byref(total)))
            cfg0 = nsd.StepOptions(gram_ns=gram, ns_steps=k).to_c()
            _lib.check(lib.dmuon_workspace_bytes(arr, 3, ctypes.byref(cfg0), ctypes.byref(base)))
            assert off.value % 256 == 0 and off.value + 12 <= total.value
            assert total.value == base.value + 256


def test_launch_info_layout_matches_header():
    assert ctypes.sizeof(_lib.LaunchInfo) == 16
    assert _lib.LaunchInfo.kind.offset == 0 and _lib.LaunchInfo.tile.offset == 4
    assert _lib.LaunchInfo.flops.offset == 8


def test_gram_and_square_launches_of_the_two_chains_merge():
    """The two chains' launches merge where they can: same kinds, and a Gram
    launch of one chain with a Square launch of the other (one launch of
    kind gram_square).  On the Llama-3.1-8B owner-0 share (direct chain for
    q_proj, Gram-space chain for the rest) this turns 23 launches into 21:
    the two q_proj Gram launches that had nothing of their kind to merge
    with share a launch with a Gram-space Square.  The executed flops are
    the two chains' own; a share with one chain only has no mixed launch."""
    L = nsd.step_launches(LLAMA8B_OWNER0, nsd.StepOptions(gram_ns=True))
    kinds = [k for k, _ in L]
    assert len(L) == 21 and kinds.count("gram_square") == 2, kinds
    q = [s for s in LLAMA8B_OWNER0 if s == (4096, 4096)]
    rest = [s for s in LLAMA8B_OWNER0 if s != (4096, 4096)]
    apart_q = nsd.step_launches(q, nsd.StepOptions(gram_ns=True))
    apart_rest = nsd.step_launches(rest, nsd.StepOptions(gram_ns=True))
    assert sum(f for _, f in L) == sum(f for _, f in apart_q) + sum(f for _, f in apart_rest)
    assert "gram_square" not in [k for k, _ in apart_q] + [k for k, _ in apart_rest]
    # each mixed launch carries a q_proj Gram (8 x m(m+1)n) and one Gram-space
    # Square over k, gate, up and down (m^2(m+1) each)
    g = 8 * 4096 * 4097 * 4096
    sq = 8 * 1024 * 1024 * 1025 + 12 * 4096 * 4096 * 4097
    assert [f for k, f in L if k == "gram_square"] == [g + sq, g + sq]
    # split launches of every kind stay well formed
    for shapes in (LLAMA8B_OWNER0, [(513, 513), (300, 700), (700, 300), (256, 1024)]):
        check_split_launches(nsd.step_launches(shapes, nsd.StepOptions(gram_ns=True)))


def test_concurrent_host_calls_agree():
    """The planner's tile-list cache is shared by every caller (a mutex
    guards it, and a full cache is cleared): host threads planning
    different shape sets at once, more sets than the cache holds, get
    the same launch sequences and workspace sizes as one thread alone."""
    import threading
    import numpy as np
    rng = np.random.default_rng(7)
    sets = []
    for _ in range(80):
        n = int(rng.integers(1, 8))
        sets.append([(int(rng.choice([17, 300, 513, 1024, 1536, 4096])),
                      int(rng.choice([33, 256, 700, 1536, 4096, 8960]))) for _ in range(n)])
    opts = [nsd.StepOptions(gram_ns=g, ns_steps=k) for g in (False, True) for k in (5, 8)]

    def plan(shapes, o):
        L = nsd.step_launches(shapes, o, tiles=True)
        arr = (_lib.Matrix * len(shapes))()
        for i, (r, c) in enumerate(shapes):
            arr[i] = _lib.Matrix(None, 0, 0, None, None, None, r, c, 1.0, 0, 0)
        out = ctypes.c_size_t(0)
        cfg = o.to_c()
        _lib.check(_lib.load().dmuon_workspace_bytes(arr, len(shapes), ctypes.byref(cfg), ctypes.byref(out)))
        return L, out.value

    want = {(i, j): plan(s, o) for i, s in enumerate(sets) for j, o in enumerate(opts)}
    got, errors = {}, []

    def worker(t):
        try:
            for rep in range(3):
                for i in range(t % 5, len(sets), 5):
                    for j, o in enumerate(opts):
                        got[(t, rep, i, j)] = plan(sets[i], o)
        except Exception as e:  # noqa: BLE001 (reported below)
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    assert len(got) == 8 * 3 * 16 * len(opts)
    for (t, rep, i, j), v in got.items():
        assert v == want[(i, j)], (t, rep, sets[i], j)


def test_chain_launch_plan():
    """DMUON_FLAG_CHAIN_LAUNCH: every bf16 product of the step is one launch
    (kind "chain", the grouped plan's flops in total, 256-tiles); matrices
    with m < 128 keep their fp32 grouped launches; the plan's waits pass the
    library's consistency check (every wait on earlier entries of the same
    XCD queue), over random shape mixes, both chains, ns_steps 1 to 8."""
    import numpy as np
    from synth import workload
    shapes = [(r, c) for _, r, c in workload(2).shapes]
    for gram in (False, True):
        grouped = nsd.step_launches(shapes, nsd.StepOptions(gram_ns=gram))
        L = nsd.step_launches(shapes, nsd.StepOptions(gram_ns=gram, chain_launch=True), tiles=True)
        assert [k for k, _, _ in L] == ["momentum_orient", "norm", "chain"]
        assert L[2][2] == 256
        assert L[2][1] == sum(f for k, f in grouped if k not in ("momentum_orient", "norm"))
    L = nsd.step_launches([(300, 700), (17, 33)], nsd.StepOptions(chain_launch=True))
    kinds = [k for k, _ in L]
    assert kinds[:3] == ["momentum_orient", "norm", "chain"] and "final" in kinds[3:]
    assert nsd.step_launches([(300, 700)], nsd.StepOptions(ns_steps=0, chain_launch=True)) == \
        nsd.step_launches([(300, 700)], nsd.StepOptions(ns_steps=0))
    rng = np.random.default_rng(3)
    for _ in range(24):
        n = int(rng.integers(1, 20))
        sh = [(int(rng.choice([1, 17, 256, 300, 513, 1024, 2000])),
               int(rng.choice([1, 33, 256, 700, 1024, 4096]))) for _ in range(n)]
        for k in (1, 2, 5, 6, 8):
            for gram in (False, True):
                o = nsd.StepOptions(ns_steps=k, gram_ns=gram, chain_launch=True)
                L = nsd.step_launches(sh, o)   # runs the consistency check
                assert sum(f for _, f in L) == sum(f for _, f in nsd.step_launches(sh, nsd.StepOptions(
                    ns_steps=k, gram_ns=gram)))


def test_chain_status_offset():
    """DMUON_FLAG_CHAIN_LAUNCH: the status word sits 4-byte aligned inside
    the workspace, after the per-XCD tickets and before its end; the offset
    call is an error without the flag, without an output pointer, and for a
    step with no chained launch (ns_steps = 0, or only fp32 matrices)."""
    lib = _lib.load()

    def call(shapes, opts, out=True):
        arr = (_lib.Matrix * len(shapes))(*[_lib.Matrix(None, 0, 0, None, None, None, r, c, 1.0, 0, 0)
                                            for r, c in shapes])
        cfg = opts.to_c()
        off, total = ctypes.c_size_t(0), ctypes.c_size_t(0)
        rc = lib.dmuon_chain_status_offset(arr, len(shapes), ctypes.byref(cfg),
                                           ctypes.byref(off) if out else None)
        if rc == _lib.OK:
            _lib.check(lib.dmuon_workspace_bytes(arr, len(shapes), ctypes.byref(cfg), ctypes.byref(total)))
        return rc, off.value, total.value

    shapes = [(300, 700), (17, 33), (513, 513)]
    for gram in (False, True):
        for k in (1, 5, 8):
            rc, off, total = call(shapes, nsd.StepOptions(ns_steps=k, gram_ns=gram, chain_launch=True))
            assert rc == _lib.OK and off % 4 == 0 and off + 4 <= total, (gram, k, off, total)
    assert call(shapes, nsd.StepOptions())[0] == _lib.ERR_INVALID_ARG
    assert call(shapes, nsd.StepOptions(chain_launch=True), out=False)[0] == _lib.ERR_INVALID_ARG
    assert call(shapes, nsd.StepOptions(ns_steps=0, chain_launch=True))[0] == _lib.ERR_INVALID_ARG
    assert call([(17, 33)], nsd.StepOptions(chain_launch=True))[0] == _lib.ERR_INVALID_ARG
