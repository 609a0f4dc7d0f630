"""Python binding of the dmuon C ABI: argument marshalling only.

Tensors are torch CUDA (HIP) tensors used as plain device memory; every step of
the Muon update runs in the HIP kernels of libdmuon.so.  Names mirror the C
entry points in include/dmuon.h.
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence

import torch

from . import _lib
from ._lib import check

_DT = {torch.float32: _lib.DMUON_F32, torch.bfloat16: _lib.DMUON_BF16}


def dtype_code(dtype: torch.dtype) -> int:
    try:
        return _DT[dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {dtype}; use torch.float32 or torch.bfloat16") from None


def _shape_arrays(shapes):
    n = len(shapes)
    rows = (ctypes.c_int64 * max(n, 1))(*[int(s[0]) for s in shapes])
    cols = (ctypes.c_int64 * max(n, 1))(*[int(s[1]) for s in shapes])
    return rows, cols


def _ptrs(tensors) -> ctypes.Array:
    n = len(tensors)
    return (ctypes.c_void_p * max(n, 1))(*[None if t is None else t.data_ptr() for t in tensors])


def _check_matrix(t: torch.Tensor, name: str, dtype: Optional[torch.dtype] = None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != 2:
        # blog post "常见错误" 2: Newton-Schulz is defined on matrices only
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


_BACKENDS = {"gram": _lib.DMUON_NS_GRAM, "direct": _lib.DMUON_NS_DIRECT}


def ns_config(ns_coeffs=None, ns_backend: str = "gram", ns_steps: Optional[int] = None):
    """A dmuon_ns_config for the given coefficients and backend, or None for the
    defaults (cubic map, gram backend).

    ns_coeffs: None (the cubic map 1.5, -0.5); one sequence (c0, c1[, c2]) used
    at every step; or ns_steps such sequences, one per step (two-term sets in a
    three-term schedule get c2 = 0).
    ns_backend: "gram" (lower-triangle Gram tiles) or "direct" (every tile).
    """
    if ns_backend not in _BACKENDS:
        raise ValueError(f"ns_backend must be 'gram' or 'direct', got {ns_backend!r}")
    if ns_coeffs is None and ns_backend == "gram":
        return None
    cfg = _lib.NsConfig()
    cfg.backend = _BACKENDS[ns_backend]
    if ns_coeffs is None:
        return cfg
    rows = list(ns_coeffs)
    if rows and all(not hasattr(c, "__len__") for c in rows):
        sets, per_step = [rows], 0
    else:
        sets, per_step = [list(r) for r in rows], 1
        if ns_steps is not None and len(sets) != ns_steps:
            raise ValueError(f"a per-step schedule needs {ns_steps} coefficient sets, got {len(sets)}")
    if not sets or any(len(r) not in (2, 3) for r in sets):
        raise ValueError("each coefficient set must hold 2 or 3 values (c0, c1[, c2])")
    n = max(len(r) for r in sets)
    # a two-term set in a three-term schedule is the same map with c2 = 0
    flat = [float(v) for r in sets for v in (list(r) + [0.0] * (n - len(r)))]
    arr = (ctypes.c_float * len(flat))(*flat)
    cfg.num_terms, cfg.per_step = n, per_step
    cfg.coeffs = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    cfg._keep = arr  # the array must outlive the struct
    return cfg


def _cfg_ptr(cfg):
    return ctypes.byref(cfg) if cfg is not None else None


def ns_workspace_bytes(shapes: Sequence[Sequence[int]], dtype: torch.dtype, ns_coeffs=None,
                       ns_backend: str = "gram") -> int:
    rows, cols = _shape_arrays(shapes)
    out = ctypes.c_size_t(0)
    cfg = ns_config(ns_coeffs, ns_backend)
    check(_lib.load().dmuon_ns_workspace_bytes(len(shapes), rows, cols, dtype_code(dtype), _cfg_ptr(cfg),
                                               ctypes.byref(out)),
          "dmuon_ns_workspace_bytes")
    return int(out.value)


def muon_step_workspace_bytes(shapes: Sequence[Sequence[int]], dtype: torch.dtype, ns_coeffs=None,
                              ns_backend: str = "gram") -> int:
    rows, cols = _shape_arrays(shapes)
    out = ctypes.c_size_t(0)
    cfg = ns_config(ns_coeffs, ns_backend)
    check(_lib.load().dmuon_muon_step_workspace_bytes(len(shapes), rows, cols, dtype_code(dtype), _cfg_ptr(cfg),
                                                      ctypes.byref(out)),
          "dmuon_muon_step_workspace_bytes")
    return int(out.value)


def muon_step_clip_workspace_bytes(shapes: Sequence[Sequence[int]], dtype: torch.dtype, num_segments: int = 1,
                                   ns_coeffs=None, ns_backend: str = "gram") -> int:
    rows, cols = _shape_arrays(shapes)
    out = ctypes.c_size_t(0)
    cfg = ns_config(ns_coeffs, ns_backend)
    check(_lib.load().dmuon_muon_step_clip_workspace_bytes(len(shapes), rows, cols, dtype_code(dtype), _cfg_ptr(cfg),
                                                           int(num_segments), ctypes.byref(out)),
          "dmuon_muon_step_clip_workspace_bytes")
    return int(out.value)


def alloc_workspace(nbytes: int, device=None) -> torch.Tensor:
    """A uint8 device buffer of at least nbytes, 256-byte aligned."""
    ws = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device or "cuda")
    if ws.data_ptr() % 256:
        raise RuntimeError("allocator returned a workspace that is not 256-byte aligned")
    return ws


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _used_on(stream, *tensors) -> None:
    """Buffers allocated here come from the caching allocator's pool of the
    current stream.  When the kernels that use them run on another stream,
    record that stream, or the block could be handed to a new allocation on
    the current stream as soon as this function drops its reference, while
    the kernels still read and write it."""
    if stream is None:
        return
    for t in tensors:
        if t is not None and stream.cuda_stream != torch.cuda.current_stream(t.device).cuda_stream:
            t.record_stream(stream)


def ns_batched(xs: Sequence[torch.Tensor], outs: Optional[Sequence[torch.Tensor]] = None, ns_steps: int = 5,
               workspace: Optional[torch.Tensor] = None, stream=None, ns_coeffs=None,
               ns_backend: str = "gram") -> List[torch.Tensor]:
    """dmuon_ns_batched: out_i = NS_{ns_steps}(x_i) for every matrix (see
    ns_config for ns_coeffs and ns_backend)."""
    if len(xs) == 0:
        return []
    dt = xs[0].dtype
    for i, x in enumerate(xs):
        _check_matrix(x, f"xs[{i}]", dt)
    own_outs = outs is None
    if own_outs:
        outs = [torch.empty_like(x) for x in xs]
    for i, (o, x) in enumerate(zip(outs, xs)):
        _check_matrix(o, f"outs[{i}]", dt)
        if o.shape != x.shape:
            raise ValueError(f"outs[{i}] shape {tuple(o.shape)} != {tuple(x.shape)}")
    shapes = [tuple(x.shape) for x in xs]
    cfg = ns_config(ns_coeffs, ns_backend, int(ns_steps))
    need = ns_workspace_bytes(shapes, dt, ns_coeffs, ns_backend)
    own_ws = workspace is None
    if own_ws:
        workspace = alloc_workspace(need, xs[0].device)
    rows, cols = _shape_arrays(shapes)
    check(_lib.load().dmuon_ns_batched(len(xs), _ptrs(xs), _ptrs(outs), rows, cols, dtype_code(dt), int(ns_steps),
                                       _cfg_ptr(cfg), ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                       ctypes.c_void_p(_stream_handle(stream))),
          "dmuon_ns_batched")
    _used_on(stream, workspace if own_ws else None, *(outs if own_outs else ()))
    return list(outs)


class MuonStep:
    """Pre-marshalled dmuon_muon_step over a fixed set of tensors.

    Builds the pointer and shape arrays once, so repeated steps (a training
    loop, the benchmark) pay only the C call.  The workspace is allocated here
    unless given.
    """

    def __init__(self, params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                 momentum: Sequence[torch.Tensor], *, ns_steps: int = 5, mu: float = 0.95, nesterov: bool = True,
                 lr: float = 0.02, lr_scale: Optional[Sequence[float]] = None, weight_decay: float = 0.0,
                 lr_scale_mode: str = "one", ns_coeffs=None, ns_backend: str = "gram",
                 update_out: Optional[Sequence[Optional[torch.Tensor]]] = None,
                 norms_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 clip_max_norm=None, clip_segments: Optional[Sequence[int]] = None, clip_norm_type: float = 2.0,
                 clip_totals: Optional[torch.Tensor] = None):
        n = len(params)
        if not (len(grads) == len(momentum) == n):
            raise ValueError("params, grads and momentum must have the same length")
        if n == 0:
            raise ValueError("empty parameter set")
        dt = params[0].dtype
        for i in range(n):
            _check_matrix(params[i], f"params[{i}]", dt)
            _check_matrix(grads[i], f"grads[{i}]", dt)
            _check_matrix(momentum[i], f"momentum[{i}]", torch.float32)
            if grads[i].shape != params[i].shape or momentum[i].shape != params[i].shape:
                raise ValueError(f"matrix {i}: params/grads/momentum shapes differ")
        if update_out is not None:
            if len(update_out) != n:
                raise ValueError("update_out must have one entry per matrix")
            for i, u in enumerate(update_out):
                if u is not None:
                    _check_matrix(u, f"update_out[{i}]", torch.float32)
                    if u.shape != params[i].shape:
                        raise ValueError(f"update_out[{i}] has the wrong shape")
        if norms_out is not None:
            if norms_out.dtype != torch.float32 or not norms_out.is_cuda or norms_out.numel() < n:
                raise ValueError("norms_out must be a float32 device tensor with one entry per matrix")
        self.count = n
        self.dtype = dt
        self.shapes = [tuple(p.shape) for p in params]
        self._keep = (list(params), list(grads), list(momentum), update_out, norms_out)
        self._params = _ptrs(params)
        self._grads = _ptrs(grads)
        self._mom = _ptrs(momentum)
        self._rows, self._cols = _shape_arrays(self.shapes)
        self._upd = _ptrs(update_out) if update_out is not None else None
        self._norms = ctypes.c_void_p(norms_out.data_ptr()) if norms_out is not None else None
        self._scale = (ctypes.c_float * n)(*[float(s) for s in lr_scale]) if lr_scale is not None else None
        self.ns_steps, self.mu, self.nesterov, self.lr = int(ns_steps), float(mu), bool(nesterov), float(lr)
        self.weight_decay = float(weight_decay)
        modes = {"one": _lib.DMUON_LR_SCALE_ONE, "moonlight": _lib.DMUON_LR_SCALE_MOONLIGHT}
        if lr_scale_mode not in modes:
            raise ValueError(f"lr_scale_mode must be 'one' or 'moonlight', got {lr_scale_mode!r}")
        self._scale_mode = modes[lr_scale_mode]
        self._cfg = ns_config(ns_coeffs, ns_backend, self.ns_steps)
        # optional clipping folded into the step (dmuon_muon_step_clipped): one
        # max norm per segment, a segment index per matrix (default all 0)
        self.clip = clip_max_norm is not None
        if self.clip:
            mn = [float(clip_max_norm)] if not hasattr(clip_max_norm, "__len__") else [float(v) for v in clip_max_norm]
            seg = [0] * n if clip_segments is None else [int(v) for v in clip_segments]
            if len(seg) != n:
                raise ValueError("clip_segments must have one entry per matrix")
            if clip_totals is not None and (clip_totals.dtype != torch.float32 or not clip_totals.is_cuda or
                                            clip_totals.numel() < len(mn)):
                raise ValueError("clip_totals must be a float32 device tensor with one entry per segment")
            self._clip_nseg = len(mn)
            self._clip_max = (ctypes.c_float * len(mn))(*mn)
            self._clip_seg = (ctypes.c_int * n)(*seg)
            self._clip_p = float(clip_norm_type)
            self._clip_totals = ctypes.c_void_p(clip_totals.data_ptr()) if clip_totals is not None else None
            self._keep = self._keep + (clip_totals,)
            self.workspace_bytes = muon_step_clip_workspace_bytes(self.shapes, dt, len(mn), ns_coeffs, ns_backend)
        else:
            self.workspace_bytes = muon_step_workspace_bytes(self.shapes, dt, ns_coeffs, ns_backend)
        self._own_ws = workspace is None
        self.workspace = workspace if workspace is not None else alloc_workspace(self.workspace_bytes,
                                                                                 params[0].device)
        if self.workspace.numel() < self.workspace_bytes:
            raise ValueError("workspace too small")
        self._lib = _lib.load()

    def __call__(self, stream=None) -> None:
        common = (self.count, self._params, self._grads, self._mom, self._rows, self._cols, dtype_code(self.dtype),
                  self.ns_steps, _cfg_ptr(self._cfg), ctypes.c_float(self.mu), 1 if self.nesterov else 0,
                  ctypes.c_float(self.lr), ctypes.c_float(self.weight_decay), self._scale_mode,
                  self._scale, self._upd, self._norms)
        tail = (ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel(),
                ctypes.c_void_p(_stream_handle(stream)))
        if self.clip:
            check(self._lib.dmuon_muon_step_clipped(*common, self._clip_seg, self._clip_nseg, self._clip_max,
                                                    ctypes.c_float(self._clip_p), self._clip_totals, *tail),
                  "dmuon_muon_step_clipped")
        else:
            check(self._lib.dmuon_muon_step(*common, *tail), "dmuon_muon_step")
        if self._own_ws:
            _used_on(stream, self.workspace)


def muon_step(params, grads, momentum, **kw) -> None:
    """dmuon_muon_step over lists of tensors (one-shot form of MuonStep)."""
    stream = kw.pop("stream", None)
    MuonStep(params, grads, momentum, **kw)(stream)


def clip_grad_norm_workspace_bytes(numels: Sequence[int], num_segments: int = 1) -> int:
    n = len(numels)
    arr = (ctypes.c_int64 * max(n, 1))(*[int(v) for v in numels])
    out = ctypes.c_size_t(0)
    check(_lib.load().dmuon_clip_grad_norm_workspace_bytes(n, arr, int(num_segments), ctypes.byref(out)),
          "dmuon_clip_grad_norm_workspace_bytes")
    return int(out.value)


def clip_grad_norm_(grads: Sequence[torch.Tensor], max_norm, segments: Optional[Sequence[int]] = None,
                    norm_type: float = 2.0, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """dmuon_clip_grad_norm: per-segment global p-norm clipping of `grads` in
    place.  `max_norm` is one float (one segment) or one per segment;
    `segments[i]` names grads[i]'s segment (default: all in segment 0).
    Returns the per-segment totals as a float32 device tensor."""
    n = len(grads)
    max_norms = [float(max_norm)] if not hasattr(max_norm, "__len__") else [float(v) for v in max_norm]
    nseg = len(max_norms)
    seg = [0] * n if segments is None else [int(v) for v in segments]
    if len(seg) != n:
        raise ValueError("segments must have one entry per gradient")
    if n == 0:
        return torch.zeros(nseg, dtype=torch.float32, device="cuda")
    dt = grads[0].dtype
    for i, g in enumerate(grads):
        if not isinstance(g, torch.Tensor) or not g.is_cuda or not g.is_contiguous() or g.dtype != dt:
            raise ValueError(f"grads[{i}] must be a contiguous device tensor of dtype {dt}")
    numel = (ctypes.c_int64 * n)(*[g.numel() for g in grads])
    segarr = (ctypes.c_int * n)(*seg)
    mn = (ctypes.c_float * nseg)(*max_norms)
    totals = torch.empty(nseg, dtype=torch.float32, device=grads[0].device)
    need = clip_grad_norm_workspace_bytes([g.numel() for g in grads], nseg)
    own_ws = workspace is None
    if own_ws:
        workspace = alloc_workspace(need, grads[0].device)
    check(_lib.load().dmuon_clip_grad_norm(n, _ptrs(grads), numel, dtype_code(dt), segarr, nseg, mn,
                                           ctypes.c_float(norm_type), ctypes.c_void_p(totals.data_ptr()),
                                           ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                           ctypes.c_void_p(_stream_handle(stream))),
          "dmuon_clip_grad_norm")
    _used_on(stream, totals, workspace if own_ws else None)
    return totals


def adamw_step_workspace_bytes(numels: Sequence[int]) -> int:
    n = len(numels)
    arr = (ctypes.c_int64 * max(n, 1))(*[int(v) for v in numels])
    out = ctypes.c_size_t(0)
    check(_lib.load().dmuon_adamw_step_workspace_bytes(n, arr, ctypes.byref(out)), "dmuon_adamw_step_workspace_bytes")
    return int(out.value)


def adamw_step_(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor], exp_avg: Sequence[torch.Tensor],
                exp_avg_sq: Sequence[torch.Tensor], step: int, lr: float = 1e-3, betas=(0.9, 0.999),
                eps: float = 1e-8, weight_decay: float = 0.01, workspace: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """dmuon_adamw_step: one AdamW step over every tensor, in place.  The
    moments are float32 tensors shaped like the parameters; `step` counts
    from 1.  Defaults are the training guide's adamw_* settings."""
    n = len(params)
    if not (len(grads) == len(exp_avg) == len(exp_avg_sq) == n):
        raise ValueError("params, grads, exp_avg and exp_avg_sq must have the same length")
    if n == 0:
        return
    dt = params[0].dtype
    for i in range(n):
        for name, t, want in (("params", params[i], dt), ("grads", grads[i], dt), ("exp_avg", exp_avg[i], torch.float32),
                              ("exp_avg_sq", exp_avg_sq[i], torch.float32)):
            if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous() or t.dtype != want:
                raise ValueError(f"{name}[{i}] must be a contiguous device tensor of dtype {want}")
            if t.numel() != params[i].numel():
                raise ValueError(f"{name}[{i}] has {t.numel()} elements, params[{i}] has {params[i].numel()}")
    numels = [p.numel() for p in params]
    numel = (ctypes.c_int64 * n)(*numels)
    own_ws = workspace is None
    if own_ws:
        workspace = alloc_workspace(adamw_step_workspace_bytes(numels), params[0].device)
    b1, b2 = betas
    check(_lib.load().dmuon_adamw_step(n, _ptrs(params), _ptrs(grads), _ptrs(exp_avg), _ptrs(exp_avg_sq), numel,
                                       dtype_code(dt), int(step), ctypes.c_float(lr), ctypes.c_float(b1),
                                       ctypes.c_float(b2), ctypes.c_float(eps), ctypes.c_float(weight_decay),
                                       ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                       ctypes.c_void_p(_stream_handle(stream))),
          "dmuon_adamw_step")
    # AdamWStep passes its own workspace and keeps it
    _used_on(stream, workspace if own_ws else None)


class AdamWStep:
    """AdamW state for a fixed list of non-matrix parameters: float32 moments
    (zeros), the step counter and a reusable workspace.  Each call runs one
    dmuon_adamw_step on the gradients given at construction."""

    def __init__(self, params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor], lr: float = 1e-3,
                 betas=(0.9, 0.999), eps: float = 1e-8, weight_decay: float = 0.01):
        self.params, self.grads = list(params), list(grads)
        self.exp_avg = [torch.zeros(p.shape, dtype=torch.float32, device=p.device) for p in self.params]
        self.exp_avg_sq = [torch.zeros(p.shape, dtype=torch.float32, device=p.device) for p in self.params]
        self.lr, self.betas, self.eps, self.weight_decay = lr, tuple(betas), eps, weight_decay
        self.step = 0
        dev = self.params[0].device if self.params else None
        self.workspace = alloc_workspace(adamw_step_workspace_bytes([p.numel() for p in self.params]), dev)

    def __call__(self, stream=None) -> None:
        self.step += 1
        adamw_step_(self.params, self.grads, self.exp_avg, self.exp_avg_sq, self.step, self.lr, self.betas,
                    self.eps, self.weight_decay, self.workspace, stream)
        _used_on(stream, self.workspace, *self.exp_avg, *self.exp_avg_sq)


def plan_summary(shapes: Sequence[Sequence[int]], dtype: torch.dtype, ns_steps: int = 5, muon: bool = True,
                 ns_coeffs=None, ns_backend: str = "gram") -> str:
    """dmuon_plan_summary: how a call over these shapes is routed, grouped and
    launched, as text (no GPU needed)."""
    rows, cols = _shape_arrays(shapes)
    cfg = ns_config(ns_coeffs, ns_backend, int(ns_steps))
    lib = _lib.load()
    need = ctypes.c_size_t(0)
    check(lib.dmuon_plan_summary(len(shapes), rows, cols, dtype_code(dtype), _cfg_ptr(cfg), int(ns_steps),
                                 1 if muon else 0, None, 0, ctypes.byref(need)), "dmuon_plan_summary")
    buf = ctypes.create_string_buffer(need.value)
    check(lib.dmuon_plan_summary(len(shapes), rows, cols, dtype_code(dtype), _cfg_ptr(cfg), int(ns_steps),
                                 1 if muon else 0, buf, need.value, None), "dmuon_plan_summary")
    return buf.value.decode()


def backend_info() -> str:
    return _lib.load().dmuon_backend_info().decode()


def profile_enable(on: bool = True) -> None:
    check(_lib.load().dmuon_profile_enable(1 if on else 0), "dmuon_profile_enable")


def profile_read() -> dict:
    """{kernel family: {launches, total_ms, flops, bytes}} since the last read."""
    stats = (_lib.KernelStat * 16)()
    n = ctypes.c_int(0)
    check(_lib.load().dmuon_profile_read(stats, 16, ctypes.byref(n)), "dmuon_profile_read")
    return {stats[i].name.decode(): dict(launches=stats[i].launches, total_ms=stats[i].total_ms,
                                         flops=stats[i].flops, bytes=stats[i].bytes) for i in range(n.value)}
