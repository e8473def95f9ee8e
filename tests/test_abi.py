"""C ABI checks that need no GPU: the library loads, exports every function
``include/dmuon.h`` declares, its host-side planning matches the oracle bit
for bit, and every argument error is reported before any HIP call (fake
device pointers are never dereferenced)."""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import partition as ref_partition
from synth import LLAMA31_8B, QWEN25_7B, model_shapes

nsd = pytest.importorskip("newton_schulz_dmuon_amd")
from newton_schulz_dmuon_amd import _lib  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_function(lib):
    header = open(os.path.join(ROOT, "include", "dmuon.h")).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(dmuon_\w+)\s*\(", header, re.M))
    assert declared == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.dmuon_abi_version() == _lib.ABI_VERSION


def test_every_export_has_a_signature(lib):
    """ctypes would otherwise truncate 64-bit pointers and sizes to int."""
    for name in _lib.EXPORTED:
        fn = getattr(lib, name)
        assert fn.restype is not None, name
        if name not in ("dmuon_abi_version", "dmuon_last_error"):
            assert fn.argtypes, name


def test_struct_layout_matches_header():
    assert ctypes.sizeof(_lib.Matrix) == 72
    assert _lib.Matrix.packed_offset.offset == 64
    assert ctypes.sizeof(_lib.StepConfig) == 32


def test_error_strings(lib):
    for code in range(0, -7, -1):
        assert lib.dmuon_error_string(code)
    assert lib.dmuon_error_string(-99) == b"unknown status"


@pytest.mark.parametrize("seed", range(20))
def test_partition_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 60))
    owners = int(rng.integers(1, 9))
    numels = [int(x) for x in rng.integers(0, 40, size=n)]  # many ties
    assert nsd.partition_lpt(numels, owners) == ref_partition.partition_lpt(numels, owners)


@pytest.mark.parametrize("shapes", [model_shapes(**LLAMA31_8B), model_shapes(**QWEN25_7B)])
@pytest.mark.parametrize("owners", [1, 3, 8])
def test_partition_model_sets_match_oracle(shapes, owners):
    numels = [r * c for _, r, c in shapes]
    assert nsd.partition_lpt(numels, owners) == ref_partition.partition_lpt(numels, owners)


@pytest.mark.parametrize("align", [1, 8, 128, 1000])
def test_pack_offsets_match_oracle(align):
    numels = [5, 0, 128, 129, 1, 77777]
    assert nsd.pack_offsets(numels, align) == ref_partition.pack_offsets(numels, align)


def test_host_call_errors(lib):
    with pytest.raises(_lib.DmuonError) as e:
        nsd.partition_lpt([1, 2], 0)
    assert e.value.status == _lib.ERR_INVALID_ARG
    with pytest.raises(_lib.DmuonError):
        nsd.partition_lpt([1, -2], 2)
    with pytest.raises(_lib.DmuonError):
        nsd.pack_offsets([1], 0)


# ------------------------------------------------ step validation, no GPU ---

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def mat(i=0, rows=8, cols=16, pdt=_lib.BF16, gdt=_lib.BF16, orth=False, base=FAKE):
    stride = 1 << 24
    b = base + i * 4 * stride
    return _lib.Matrix(b, pdt, gdt, b + stride, b + 2 * stride, b + 3 * stride if orth else None,
                       rows, cols, 1.0, 0, 0)


def cfg(**kw):
    c = dict(a=3.4445, b=-4.775, c=2.0315, ns_steps=5, lr=0.02, momentum=0.95, eps=1e-7, flags=0)
    c.update(kw)
    return _lib.StepConfig(c["a"], c["b"], c["c"], c["ns_steps"], c["lr"], c["momentum"],
                           c["eps"], c["flags"])


def ws_bytes(lib, mats, c):
    arr = (_lib.Matrix * len(mats))(*mats)
    out = ctypes.c_size_t(0)
    rc = lib.dmuon_workspace_bytes(arr, len(mats), ctypes.byref(c), ctypes.byref(out))
    return rc, out.value


def step(lib, mats, c, ws=FAKE + (1 << 40), nbytes=None):
    arr = (_lib.Matrix * max(len(mats), 1))(*mats)
    if nbytes is None:
        nbytes = ws_bytes(lib, mats, c)[1]
    return lib.dmuon_muon_step(arr, len(mats), ctypes.byref(c), ws, nbytes, None)


def test_zero_matrices_is_noop(lib):
    assert step(lib, [], cfg(), ws=None, nbytes=0) == _lib.OK


def test_workspace_size_grows_with_shape(lib):
    rc1, b1 = ws_bytes(lib, [mat(rows=8, cols=16)], cfg())
    rc2, b2 = ws_bytes(lib, [mat(rows=300, cols=700)], cfg())
    rc3, b3 = ws_bytes(lib, [mat(rows=300, cols=700)], cfg(flags=_lib.FLAG_NS_FP32))
    rc4, b4 = ws_bytes(lib, [mat(rows=300, cols=700)], cfg(ns_steps=0))
    assert rc1 == rc2 == rc3 == rc4 == _lib.OK
    assert b1 < b2 < b3 and b4 < b2
    # 300 x 700 pads to 512 x 768: 2 X^T buffers + A + B in bf16 at least
    assert b2 >= 2 * (2 * 512 * 768 + 2 * 512 * 512)


@pytest.mark.parametrize("bad,code", [
    (dict(ns_steps=-1), _lib.ERR_INVALID_ARG),
    (dict(ns_steps=65), _lib.ERR_INVALID_ARG),
    (dict(lr=float("nan")), _lib.ERR_INVALID_ARG),
    (dict(momentum=float("inf")), _lib.ERR_INVALID_ARG),
    (dict(eps=-1.0), _lib.ERR_INVALID_ARG),
    (dict(flags=1 << 7), _lib.ERR_INVALID_ARG),
])
def test_bad_config(lib, bad, code):
    assert step(lib, [mat()], cfg(**bad), nbytes=1 << 30) == code


def test_step_side_limit(lib):
    """The step takes at most 2^22 elements per side (the kernels' 32-bit
    row-block offsets and 16-bit tile indices); pack and unpack do not."""
    c = cfg()
    ok = mat(rows=1 << 22, cols=2)
    rc, _ = ws_bytes(lib, [ok], c)
    assert rc == _lib.OK
    for r, cc in ((1 << 22) + 1, 2), (2, (1 << 22) + 1):
        m = mat(rows=r, cols=cc)
        rc, _ = ws_bytes(lib, [m], c)
        assert rc == _lib.ERR_INVALID_ARG
        assert step(lib, [m], c, nbytes=1 << 30) == _lib.ERR_INVALID_ARG
        assert b"limit" in lib.dmuon_last_error()


def test_bad_matrices(lib):
    c = cfg()
    big = 1 << 30
    m = mat(); m.rows = 0
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_INVALID_ARG
    m = mat(); m.cols = -3
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_INVALID_ARG
    m = mat(); m.param_dtype = 7
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_UNSUPPORTED_DTYPE
    m = mat(); m.reserved = 1
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_INVALID_ARG
    m = mat(); m.scale = float("nan")
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_INVALID_ARG
    m = mat(); m.param = None
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_INVALID_ARG
    m = mat(); m.momentum = None
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_INVALID_ARG
    m = mat(); m.grad = FAKE + 8
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_MISALIGNED
    assert lib.dmuon_muon_step(None, 1, ctypes.byref(c), FAKE, big, None) == _lib.ERR_INVALID_ARG
    arr = (_lib.Matrix * 1)(mat())
    assert lib.dmuon_muon_step(arr, 1, None, FAKE, big, None) == _lib.ERR_INVALID_ARG
    assert lib.dmuon_muon_step(arr, -1, ctypes.byref(c), FAKE, big, None) == _lib.ERR_INVALID_ARG


def test_workspace_errors(lib):
    c = cfg()
    need = ws_bytes(lib, [mat()], c)[1]
    assert step(lib, [mat()], c, nbytes=need - 1) == _lib.ERR_WORKSPACE_TOO_SMALL
    assert step(lib, [mat()], c, ws=None, nbytes=need) == _lib.ERR_INVALID_ARG
    assert step(lib, [mat()], c, ws=FAKE + (1 << 40) + 16, nbytes=need) == _lib.ERR_MISALIGNED
    # workspace overlapping a parameter
    assert step(lib, [mat()], c, ws=FAKE, nbytes=need) == _lib.ERR_ALIAS


def test_alias_errors(lib):
    c = cfg()
    big = 1 << 30
    m = mat(); m.momentum = m.param                         # written twice
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_ALIAS
    m = mat(); m.grad = m.momentum                          # read overlaps written
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_ALIAS
    a, b = mat(0), mat(1)
    b.param = a.param + 64                                   # two params overlap
    assert step(lib, [a, b], c, nbytes=big) == _lib.ERR_ALIAS
    a, b = mat(0), mat(1)
    b.grad = a.grad                                          # shared read-only grad is fine:
    # it passes the alias check and stops at the (deliberately) small workspace
    assert step(lib, [a, b], c, nbytes=1) == _lib.ERR_WORKSPACE_TOO_SMALL
    m = mat(orth=True); m.orth_out = m.grad
    assert step(lib, [m], c, nbytes=big) == _lib.ERR_ALIAS


def test_pack_errors(lib):
    m = mat(rows=4, cols=8)
    m.packed_offset = 0
    arr = (_lib.Matrix * 1)(m)
    packed = FAKE + (1 << 40)
    assert lib.dmuon_pack(arr, 1, 5, packed, _lib.BF16, 32, None) == _lib.ERR_INVALID_ARG
    assert lib.dmuon_pack(arr, 1, 0, packed, _lib.F32, 32, None) == _lib.ERR_UNSUPPORTED_DTYPE
    assert lib.dmuon_pack(arr, 1, 0, packed, _lib.BF16, 31, None) == _lib.ERR_INVALID_ARG
    assert lib.dmuon_pack(arr, 1, 0, None, _lib.BF16, 32, None) == _lib.ERR_INVALID_ARG
    m.packed_offset = 3
    arr = (_lib.Matrix * 1)(m)
    assert lib.dmuon_pack(arr, 1, 0, packed, _lib.BF16, 64, None) == _lib.ERR_MISALIGNED
    a, b = mat(0, 4, 8), mat(1, 4, 8)
    a.packed_offset, b.packed_offset = 0, 16             # overlap in the packed buffer
    arr = (_lib.Matrix * 2)(a, b)
    assert lib.dmuon_pack(arr, 2, 0, packed, _lib.BF16, 64, None) == _lib.ERR_ALIAS
    m = mat(0, 4, 8)
    arr = (_lib.Matrix * 1)(m)                            # packed over the source param
    assert lib.dmuon_pack(arr, 1, 0, m.param, _lib.BF16, 64, None) == _lib.ERR_ALIAS
    assert lib.dmuon_pack(arr, 0, 0, packed, _lib.BF16, 0, None) == _lib.OK


def test_step_packed_errors(lib):
    """Argument errors of dmuon_muon_step_packed, all reported before any HIP
    call; valid slots pass every packed check and stop at the small workspace."""
    c = cfg()
    packed = FAKE + (1 << 41)

    def sp(mats, packed=packed, pdt=_lib.BF16, numel=1 << 20, nbytes=1):
        arr = (_lib.Matrix * max(len(mats), 1))(*mats)
        return lib.dmuon_muon_step_packed(arr, len(mats), ctypes.byref(c), FAKE + (1 << 40), nbytes,
                                          packed, pdt, numel, None, None, 0)

    a, b = mat(0), mat(1)                     # 8 x 16 = 128 elements each
    a.packed_offset, b.packed_offset = 0, 128
    assert sp([a, b]) == _lib.ERR_WORKSPACE_TOO_SMALL
    assert sp([a, b], packed=None) == _lib.ERR_INVALID_ARG
    assert sp([a, b], pdt=_lib.F32) == _lib.ERR_UNSUPPORTED_DTYPE   # params are bf16
    assert sp([a, b], pdt=9) == _lib.ERR_UNSUPPORTED_DTYPE
    assert sp([a, b], numel=255) == _lib.ERR_INVALID_ARG             # b's slot runs past the end
    assert sp([a, b], numel=-1) == _lib.ERR_INVALID_ARG
    b.packed_offset = 100                                             # 200 bytes: misaligned
    assert sp([a, b]) == _lib.ERR_MISALIGNED
    b.packed_offset = 64                                              # overlaps a's slot
    assert sp([a, b]) == _lib.ERR_ALIAS
    m = mat(0)
    assert sp([m], packed=m.grad) == _lib.ERR_ALIAS                   # slot over a read buffer
    assert sp([m], packed=m.param + 128) == _lib.ERR_ALIAS            # slot over the param
    m.packed_offset = -8
    assert sp([m]) == _lib.ERR_INVALID_ARG
    assert sp([], nbytes=0) == _lib.OK


# ------------------------------------------------ AdamW validation, no GPU ---

def tensor(i=0, numel=100, pdt=_lib.BF16, gdt=_lib.BF16):
    stride = 1 << 24
    b = FAKE + (i + 16) * 4 * stride
    return _lib.Tensor(b, pdt, gdt, b + stride, b + 2 * stride, b + 3 * stride, numel)


def adam(lib, ts, **kw):
    c = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)
    c.update(kw)
    cfg = _lib.AdamWConfig(c["lr"], c["beta1"], c["beta2"], c["eps"], c["weight_decay"], c["step"])
    arr = (_lib.Tensor * max(len(ts), 1))(*ts)
    return lib.dmuon_adamw_step(arr, len(ts), ctypes.byref(cfg), None)


def test_adamw_struct_layout():
    assert ctypes.sizeof(_lib.Tensor) == 48
    assert ctypes.sizeof(_lib.AdamWConfig) == 24


def test_adamw_errors(lib):
    assert adam(lib, []) == _lib.OK
    for bad in (dict(step=0), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0),
                dict(lr=float("nan")), dict(weight_decay=float("inf"))):
        assert adam(lib, [tensor()], **bad) == _lib.ERR_INVALID_ARG, bad
    t = tensor(); t.numel = 0
    assert adam(lib, [t]) == _lib.ERR_INVALID_ARG
    t = tensor(); t.param_dtype = 3
    assert adam(lib, [t]) == _lib.ERR_UNSUPPORTED_DTYPE
    t = tensor(); t.exp_avg = None
    assert adam(lib, [t]) == _lib.ERR_INVALID_ARG
    t = tensor(); t.exp_avg_sq = t.exp_avg_sq + 4
    assert adam(lib, [t]) == _lib.ERR_MISALIGNED
    t = tensor(); t.exp_avg_sq = t.exp_avg
    assert adam(lib, [t]) == _lib.ERR_ALIAS
    a, b = tensor(0), tensor(1)
    b.param = a.grad
    assert adam(lib, [a, b]) == _lib.ERR_ALIAS
