"""Python face of ``libdmuon.so`` over torch tensors.

PyTorch only supplies device memory and the current HIP stream; every step of
the owner's Muon update runs in the library's HIP kernels.  Each function
here only fills the C structs and checks the returned status.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

from . import _lib
from ._lib import AdamWConfig, DmuonError, LaunchInfo, Matrix, StepConfig, Tensor, check, load

# Public Muon quintic (Jordan et al., 2024); the DMuon pages print none.
QUINTIC = (3.4445, -4.7750, 2.0315)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    raise DmuonError(_lib.ERR_UNSUPPORTED_DTYPE, f"tensor dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise DmuonError(_lib.ERR_INVALID_ARG, "tensors must be contiguous")
    return t.data_ptr()


def _stream_handle(device, stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _keep_for_stream(t, device, stream) -> None:
    """PyTorch's caching allocator ties a block to the stream that allocated
    it and may hand it out again as soon as the tensor is freed.  A buffer
    allocated on the current stream but used by kernels on another one is
    marked as in use by that stream too, so that neither its release (a
    temporary workspace) nor its replacement (a growing Workspace) lets a
    new tensor take the memory before those kernels are done."""
    import torch
    if stream is not None and stream != torch.cuda.current_stream(device):
        t.record_stream(stream)


@dataclass
class StepOptions:
    """``dmuon_step_config``.  ``lr`` and ``ns_steps`` defaults are the ones in
    the DMuon landing page's optimizer call ("LLM Pretraining")."""

    a: float = QUINTIC[0]
    b: float = QUINTIC[1]
    c: float = QUINTIC[2]
    ns_steps: int = 5
    lr: float = 0.02
    momentum: float = 0.95
    eps: float = 1e-7
    nesterov: bool = False
    ns_fp32: bool = False
    # Gram-space chain for matrices with max(r,c) >= 2 min(r,c) (see
    # DMUON_FLAG_GRAM_NS); the others keep the direct chain.  Fewer flops,
    # as accurate on Gaussian gradients, 2-3x less accurate when the
    # singular values spread over one or two decades
    gram_ns: bool = False
    # record per matrix whether U holds a NaN or an Inf (nonfinite_flags)
    check_finite: bool = False
    # every bf16 product of the step in one dependency-driven launch (see
    # DMUON_FLAG_CHAIN_LAUNCH)
    chain_launch: bool = False

    def to_c(self) -> StepConfig:
        flags = (_lib.FLAG_NESTEROV if self.nesterov else 0) | \
                (_lib.FLAG_NS_FP32 if self.ns_fp32 else 0) | \
                (_lib.FLAG_GRAM_NS if self.gram_ns else 0) | \
                (_lib.FLAG_CHECK_FINITE if self.check_finite else 0) | \
                (_lib.FLAG_CHAIN_LAUNCH if self.chain_launch else 0)
        return StepConfig(self.a, self.b, self.c, int(self.ns_steps), self.lr,
                          self.momentum, self.eps, flags)


def matrices(params, grads=None, momenta=None, scales=None, orth_out=None,
             packed_offsets=None):
    """Builds the ``dmuon_matrix`` array from parallel tensor lists."""
    n = len(params)
    arr = (Matrix * max(n, 1))()
    for i in range(n):
        p = params[i]
        if p.dim() != 2:
            raise DmuonError(_lib.ERR_INVALID_ARG, f"matrix {i} is not 2-D")
        g = grads[i] if grads is not None else None
        m = momenta[i] if momenta is not None else None
        o = orth_out[i] if orth_out is not None else None
        arr[i] = Matrix(
            _ptr(p), _dtype_code(p), _dtype_code(g) if g is not None else _dtype_code(p),
            _ptr(g), _ptr(m), _ptr(o), p.shape[0], p.shape[1],
            float(scales[i]) if scales is not None else 1.0, 0,
            int(packed_offsets[i]) if packed_offsets is not None else 0)
    return arr, n


def step_launches(shapes: Sequence, opts: StepOptions, tiles: bool = False):
    """The step's launch sequence for matrices of these ``(rows, cols)``
    shapes: a list of ``(kind, algorithmic_flops)``, kind a name from
    ``_lib.LAUNCH_KINDS``; with ``tiles``, ``(kind, flops, tile_edge)``
    (0 for the element-wise launches).  Host-only."""
    n = len(shapes)
    arr = (Matrix * max(n, 1))()
    for i, (r, c) in enumerate(shapes):
        arr[i] = Matrix(None, _lib.BF16, _lib.BF16, None, None, None, int(r), int(c), 1.0, 0, 0)
    cfg = opts.to_c()
    lib = load()
    count = ctypes.c_int32(0)
    check(lib.dmuon_step_launches(arr, n, ctypes.byref(cfg), None, 0, ctypes.byref(count)))
    out = (LaunchInfo * max(count.value, 1))()
    check(lib.dmuon_step_launches(arr, n, ctypes.byref(cfg), out, count.value, ctypes.byref(count)))
    if tiles:
        return [(_lib.LAUNCH_KINDS[out[j].kind], out[j].flops, out[j].tile) for j in range(count.value)]
    return [(_lib.LAUNCH_KINDS[out[j].kind], out[j].flops) for j in range(count.value)]


def nonfinite_flags(params, opts: StepOptions, workspace: Workspace):
    """The per-matrix flags a step with ``opts.check_finite`` wrote into
    ``workspace``: a device int32 tensor, 1 where that matrix's U held a NaN
    or an Inf.  A view of the workspace; read it after the step's stream has
    synchronised and before the workspace is used again."""
    import torch
    arr, n = matrices(params)
    off = ctypes.c_size_t(0)
    cfg = opts.to_c()
    check(load().dmuon_nonfinite_flags_offset(arr, n, ctypes.byref(cfg), ctypes.byref(off)))
    return workspace.buf[off.value:off.value + 4 * n].view(torch.int32)


def chain_status(params, opts: StepOptions, workspace: Workspace):
    """The status word a step with ``opts.chain_launch`` left in
    ``workspace``: a one-element device int32 tensor, 1 if a wait of the
    chained launch gave up (that step's result is wrong), else 0.  A view of
    the workspace; read it after the step's stream has synchronised and
    before the workspace is used again."""
    import torch
    arr, n = matrices(params)
    off = ctypes.c_size_t(0)
    cfg = opts.to_c()
    check(load().dmuon_chain_status_offset(arr, n, ctypes.byref(cfg), ctypes.byref(off)))
    return workspace.buf[off.value:off.value + 4].view(torch.int32)


def workspace_bytes(params, opts: StepOptions) -> int:
    arr, n = matrices(params)
    out = ctypes.c_size_t(0)
    cfg = opts.to_c()
    check(load().dmuon_workspace_bytes(arr, n, ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


class Workspace:
    """Device scratch for ``muon_step``, grown on demand (PyTorch allocates)."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device):
        import torch
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = None
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


def muon_step(params: Sequence, grads: Sequence, momenta: Sequence, scales: Sequence[float],
              opts: StepOptions = StepOptions(), orth_out: Optional[Sequence] = None,
              workspace: Optional[Workspace] = None, stream=None, packed=None,
              packed_offsets: Optional[Sequence[int]] = None) -> None:
    """One owner-side Muon step over the matrices, in place on ``params`` and
    ``momenta`` (and ``orth_out`` when given).  With ``packed`` (and the
    matrices' ``packed_offsets``), the updated params are also written into
    that buffer, as ``pack`` would right after the step.  Enqueued on
    ``stream`` (the current stream by default); synchronise before reading
    the results."""
    n = len(params)
    if n == 0:
        return
    device = params[0].device
    if (packed is None) != (packed_offsets is None):
        raise DmuonError(_lib.ERR_INVALID_ARG, "packed and packed_offsets go together")
    arr, n = matrices(params, grads, momenta, scales, orth_out, packed_offsets)
    cfg = opts.to_c()
    lib = load()
    need = ctypes.c_size_t(0)
    check(lib.dmuon_workspace_bytes(arr, n, ctypes.byref(cfg), ctypes.byref(need)))
    ws = (workspace or Workspace()).get(need.value, device)
    _keep_for_stream(ws, device, stream)
    if packed is None:
        check(lib.dmuon_muon_step(arr, n, ctypes.byref(cfg), ws.data_ptr(), ws.numel(),
                                  _stream_handle(device, stream)))
    else:
        check(lib.dmuon_muon_step_packed(arr, n, ctypes.byref(cfg), ws.data_ptr(), ws.numel(),
                                         _ptr(packed), _dtype_code(packed), packed.numel(),
                                         _stream_handle(device, stream), None, 0))


def muon_step_noalloc(params: Sequence, grads: Sequence, momenta: Sequence,
                      scales: Sequence[float], opts: StepOptions = StepOptions(),
                      orth_out: Optional[Sequence] = None, stream=None) -> None:
    """``muon_step`` without a workspace: ``dmuon_muon_step_noalloc`` works
    in the library's static per-device scratch (``_lib.NOALLOC_SCRATCH_BYTES``)
    and allocates nothing.  Calls overlapping on one GPU race on that
    scratch; calls in stream order are safe."""
    n = len(params)
    if n == 0:
        return
    arr, n = matrices(params, grads, momenta, scales, orth_out)
    cfg = opts.to_c()
    check(load().dmuon_muon_step_noalloc(arr, n, ctypes.byref(cfg),
                                         _stream_handle(params[0].device, stream)))


def pack(tensors: Sequence, offsets: Sequence[int], packed, stream=None) -> None:
    """``packed[offsets[i] + r*cols + c] = tensors[i][r, c]`` (bit copy)."""
    arr, n = matrices(tensors, packed_offsets=offsets)
    check(load().dmuon_pack(arr, n, _lib.FIELD_PARAM, _ptr(packed), _dtype_code(packed),
                            packed.numel(), _stream_handle(packed.device, stream)))


def unpack(packed, tensors: Sequence, offsets: Sequence[int], stream=None) -> None:
    """``tensors[i][r, c] = packed[offsets[i] + r*cols + c]`` (bit copy)."""
    arr, n = matrices(tensors, packed_offsets=offsets)
    check(load().dmuon_unpack(arr, n, _lib.FIELD_PARAM, _ptr(packed), _dtype_code(packed),
                              packed.numel(), _stream_handle(packed.device, stream)))


def partition_lpt(numels: Sequence[int], n_owners: int):
    """Balanced ownership: ``(owner_of_matrix, load_of_owner)``."""
    n = len(numels)
    arr = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in numels])
    owners = (ctypes.c_int32 * max(n, 1))()
    loads = (ctypes.c_int64 * max(n_owners, 1))()
    check(load().dmuon_partition_lpt(arr, n, n_owners, owners, loads))
    return list(owners[:n]), list(loads[:max(n_owners, 0)])


def pack_offsets(numels: Sequence[int], align: int = 128):
    """Aligned offsets of consecutive matrices in one buffer: ``(offsets, total)``."""
    n = len(numels)
    arr = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in numels])
    offs = (ctypes.c_int64 * max(n, 1))()
    total = ctypes.c_int64(0)
    check(load().dmuon_pack_offsets(arr, n, int(align), offs, ctypes.byref(total)))
    return list(offs[:n]), total.value


@dataclass
class AdamWOptions:
    """``dmuon_adamw_config``; ``lr`` default is the landing page's
    ``adamw_lr`` (1e-3), the rest are not on the pages (PyTorch's AdamW
    defaults)."""

    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01

    def to_c(self, step: int) -> AdamWConfig:
        return AdamWConfig(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay, int(step))


def adamw_step(params: Sequence, grads: Sequence, exp_avgs: Sequence, exp_avg_sqs: Sequence,
               step: int, opts: AdamWOptions = AdamWOptions(), stream=None) -> None:
    """AdamW on the non-Muon parameters, in place (tensors of any shape)."""
    n = len(params)
    if n == 0:
        return
    arr = (Tensor * n)()
    for i in range(n):
        p, g = params[i], grads[i]
        arr[i] = Tensor(_ptr(p), _dtype_code(p), _dtype_code(g), _ptr(g), _ptr(exp_avgs[i]),
                        _ptr(exp_avg_sqs[i]), p.numel())
    cfg = opts.to_c(step)
    check(load().dmuon_adamw_step(arr, n, ctypes.byref(cfg),
                                  _stream_handle(params[0].device, stream)))
