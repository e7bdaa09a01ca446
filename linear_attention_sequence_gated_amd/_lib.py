"""ctypes binding of libkda.so: argument marshalling only.

Every step of the KDA path runs in the library's HIP kernels; this module
checks tensor shapes, allocates outputs and the workspace through PyTorch
(device memory and streams are all PyTorch is used for here) and forwards
raw pointers to the C ABI declared in include/kda.h.  There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import build as _build

KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED", 3: "KDA_ERR_WORKSPACE",
           4: "KDA_ERR_HIP", 5: "KDA_ERR_RANGE"}
KDA_ERR_RANGE = 5
KDA_ERR_INVALID_ARG = 1

# Every symbol include/kda.h declares.
EXPORTED = ("kda_status_string", "kda_chunk_fwd_workspace_size", "kda_chunk_fwd", "kda_chunk_fwd_intra",
            "kda_chunk_fwd_inter", "kda_chunk_fwd_ex", "kda_chunk_fwd_ex_workspace_size", "kda_decode_step",
            "kda_decode_step_ex", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_status", "kda_chunk_fwd_plan",
            "kda_chunk_fwd_windowed", "kda_chunk_fwd_windowed_ex")
# Bytes of the library-held scratch of kda_chunk_fwd_noalloc (KDA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


class ChunkParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int64), ("num_seqs", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim_k", ctypes.c_int32),
                ("head_dim_v", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
                ("scale", ctypes.c_float), ("qkv_dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32)]


class ChunkPlan(ctypes.Structure):
    """kda_chunk_plan_t (include/kda.h)."""
    _fields_ = [("chunk_size", ctypes.c_int32), ("whole_rows", ctypes.c_int32),
                ("range_chunks", ctypes.c_int32), ("max_ranges", ctypes.c_int32)]


class ChunkOptions(ctypes.Structure):
    """kda_chunk_options_t (include/kda.h); zero-filled = the plain operation."""
    _fields_ = [("checkpoints", ctypes.c_void_p), ("ckpt_every", ctypes.c_int64), ("max_ckpts", ctypes.c_int32),
                ("decay_floor", ctypes.c_float), ("alpha_mode", ctypes.c_int32), ("fuse_inputs", ctypes.c_int32),
                ("gate", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float)]


class DecodeOptions(ctypes.Structure):
    """kda_decode_options_t (include/kda.h); zero-filled = the plain step."""
    _fields_ = [("state_slots", ctypes.c_void_p), ("decay_floor", ctypes.c_float), ("alpha_mode", ctypes.c_int32),
                ("fuse_inputs", ctypes.c_int32), ("gate", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("pool_entries", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return _build.LIB


def load() -> ctypes.CDLL:
    """Load libkda.so (built in-tree); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("KDA_LIBRARY", _build.LIB)   # another build of the same ABI
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(python -m linear_attention_sequence_gated_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_int
    lib.kda_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(ChunkParams), ctypes.POINTER(sz)]
    lib.kda_chunk_fwd_plan.restype = ctypes.c_int
    lib.kda_chunk_fwd_plan.argtypes = [ctypes.POINTER(ChunkParams), i32, ctypes.POINTER(ChunkPlan)]
    for name in ("kda_chunk_fwd", "kda_chunk_fwd_intra", "kda_chunk_fwd_inter"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.POINTER(ChunkParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd_ex_workspace_size.restype = ctypes.c_int
    lib.kda_chunk_fwd_ex_workspace_size.argtypes = [ctypes.POINTER(ChunkParams), ctypes.POINTER(ChunkOptions),
                                                    ctypes.POINTER(sz)]
    lib.kda_chunk_fwd_ex.restype = ctypes.c_int
    lib.kda_chunk_fwd_ex.argtypes = [ctypes.POINTER(ChunkParams), ctypes.POINTER(ChunkOptions),
                                     vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kda_chunk_fwd_status.restype = ctypes.c_int
    lib.kda_chunk_fwd_status.argtypes = [vp, vp]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_chunk_fwd_windowed.restype = ctypes.c_int
    lib.kda_chunk_fwd_windowed.argtypes = [ctypes.POINTER(ChunkParams), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           sz, vp]
    lib.kda_chunk_fwd_windowed_ex.restype = ctypes.c_int
    lib.kda_chunk_fwd_windowed_ex.argtypes = [ctypes.POINTER(ChunkParams), ctypes.POINTER(ChunkOptions),
                                              vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [i32, i32, i32, i32, f32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kda_decode_step_ex.restype = ctypes.c_int
    lib.kda_decode_step_ex.argtypes = [i32, i32, i32, i32, f32, i32, i32, ctypes.POINTER(DecodeOptions),
                                       vp, vp, vp, vp, vp, vp, vp, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().kda_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KdaError(fn, status, status_string(status))


def _code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return KDA_DTYPE_BF16
    if dtype == torch.float32:
        return KDA_DTYPE_F32
    raise TypeError(f"q/k/v and o must be bfloat16 or float32, got {dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(cond: bool, what: str) -> None:
    if not cond:
        raise ValueError(what)


def _on_device(t: torch.Tensor) -> bool:
    """Whether `t` lives in device memory (the kernels dereference every pointer on the GPU)."""
    return t.is_cuda


def _dense(t: Optional[torch.Tensor], shape, dtype, what: str) -> None:
    """`t` is None or a contiguous device tensor of exactly `shape` and `dtype`."""
    if t is None:
        return
    _need(tuple(t.shape) == tuple(shape) and t.dtype == dtype and _on_device(t) and t.is_contiguous(),
          f"{what} must be a contiguous {dtype} device tensor of shape {tuple(shape)}, got "
          f"{tuple(t.shape)} {t.dtype} on {t.device}{'' if t.is_contiguous() else ' (strided)'}")


def chunk_params(q: torch.Tensor, v: torch.Tensor, cu_seqlens: Optional[torch.Tensor],
                 chunk_size: int, scale: float, o_dtype: Optional[torch.dtype] = None) -> ChunkParams:
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    n = B if cu_seqlens is None else cu_seqlens.numel() - 1
    return ChunkParams(B, T, n, H, dk, dv, chunk_size, scale, _code(q.dtype),
                       _code(q.dtype if o_dtype is None else o_dtype))


def workspace_size(q: torch.Tensor, v: torch.Tensor, cu_seqlens=None, chunk_size: int = 64,
                   scale: float = 1.0) -> int:
    p = chunk_params(q, v, cu_seqlens, chunk_size, scale)
    out = ctypes.c_size_t(0)
    _check("kda_chunk_fwd_workspace_size", load().kda_chunk_fwd_workspace_size(ctypes.byref(p),
                                                                              ctypes.byref(out)))
    return out.value


def chunk_plan(q: torch.Tensor, v: torch.Tensor, cu_seqlens=None, chunk_size: int = 64) -> dict:
    """How kda_chunk_fwd runs a call of this shape on the current device
    (kda_chunk_fwd_plan): chunk_size, whole_rows, range_chunks, max_ranges."""
    p = chunk_params(q, v, cu_seqlens, chunk_size, 1.0)
    out = ChunkPlan()
    _check("kda_chunk_fwd_plan", load().kda_chunk_fwd_plan(ctypes.byref(p), int(cu_seqlens is not None),
                                                          ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in ChunkPlan._fields_}


def _check_options(q, v, n, checkpoints, ckpt_every, gate, norm_weight) -> None:
    """Shapes of the option tensors of a prefill call with N = n sequences."""
    _, _, H, dk = q.shape
    dv = v.shape[-1]
    if ckpt_every:
        _need(checkpoints is not None and checkpoints.dim() == 5 and checkpoints.shape[0] == n
              and checkpoints.shape[2:] == (H, dk, dv) and checkpoints.dtype == torch.float32
              and _on_device(checkpoints) and checkpoints.is_contiguous(),
              "checkpoints must be fp32 [N, max_ckpts, H, dk, dv]")
    _dense(gate, v.shape, q.dtype, "gate")
    _dense(norm_weight, (v.shape[-1],), torch.float32, "norm_weight")


def _chunk_options(checkpoints, ckpt_every, decay_floor, alpha_scalar, fuse_inputs, gate, norm_weight,
                   norm_eps) -> Optional[ChunkOptions]:
    """kda_chunk_options_t of the keyword options (None: the plain call)."""
    if not (ckpt_every or decay_floor or alpha_scalar or fuse_inputs or gate is not None
            or norm_weight is not None):
        return None
    return ChunkOptions(checkpoints=checkpoints.data_ptr() if ckpt_every else None,
                        ckpt_every=int(ckpt_every),
                        max_ckpts=checkpoints.shape[1] if ckpt_every else 0,
                        decay_floor=float(decay_floor), alpha_mode=int(bool(alpha_scalar)),
                        fuse_inputs=int(bool(fuse_inputs)),
                        gate=None if gate is None else gate.data_ptr(),
                        norm_weight=None if norm_weight is None else norm_weight.data_ptr(),
                        norm_eps=float(norm_eps))


class Prefill:
    """A kda_chunk_fwd call with its arguments marshalled once.

    ``run()`` issues kda_chunk_fwd (kda_chunk_fwd_ex with options);
    ``intra()`` / ``inter()`` issue the two halves of a plain call and raise
    ValueError for a call with options.  The tensors are kept alive by this
    object.
    """

    def __init__(self, q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, chunk_size: int = 64,
                 scale: float = 1.0, output_final_state: bool = True, o=None, final_state=None,
                 workspace=None, stream=None, o_dtype: Optional[torch.dtype] = None,
                 checkpoints=None, ckpt_every: int = 0, decay_floor: float = 0.0,
                 alpha_scalar: bool = False, fuse_inputs: bool = False, gate=None, norm_weight=None,
                 norm_eps: float = 0.0):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        _need(k.shape == q.shape, "q and k must share [B,T,H,dk]")
        _need(alpha.shape == ((B, T, H) if alpha_scalar else q.shape),
              "alpha must be [B,T,H,dk] ([B,T,H] with alpha_scalar)")
        _need(v.shape == (B, T, H, dv) and beta.shape == (B, T, H), "v/beta shapes")
        _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
        _need(alpha.dtype == torch.float32 and beta.dtype == torch.float32, "alpha, beta must be fp32")
        for t in (q, k, v, alpha, beta):
            _need(_on_device(t) and t.is_contiguous(), "inputs must be contiguous device tensors")
        if cu_seqlens is not None:
            _need(cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2,
                  "cu_seqlens must be int32 [N+1] with N >= 1")
            _dense(cu_seqlens, (cu_seqlens.numel(),), torch.int32, "cu_seqlens")
        n = B if cu_seqlens is None else cu_seqlens.numel() - 1
        _dense(initial_state, (n, H, dk, dv), torch.float32, "initial_state")
        _dense(final_state, (n, H, dk, dv), torch.float32, "final_state")
        o_dtype = q.dtype if o_dtype is None else o_dtype
        _dense(o, v.shape, o_dtype, "o")
        _check_options(q, v, n, checkpoints, ckpt_every, gate, norm_weight)
        # every check above precedes the first allocation
        if o is None:
            o = torch.empty(v.shape, dtype=o_dtype, device=v.device)
        if final_state is None and output_final_state:
            final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device)
        self.params = chunk_params(q, v, cu_seqlens, chunk_size, scale, o_dtype)
        self.o, self.final_state = o, final_state
        self.checkpoints = checkpoints
        self.options = _chunk_options(checkpoints, ckpt_every, decay_floor, alpha_scalar, fuse_inputs, gate,
                                      norm_weight, norm_eps)
        out = ctypes.c_size_t(0)
        _check("kda_chunk_fwd_ex_workspace_size",
               load().kda_chunk_fwd_ex_workspace_size(ctypes.byref(self.params),
                                                      None if self.options is None else ctypes.byref(self.options),
                                                      ctypes.byref(out)))
        if workspace is None:
            workspace = torch.empty(max(out.value, 1), dtype=torch.uint8, device=q.device)
        self.workspace = workspace
        self._keep = (q, k, v, alpha, beta, initial_state, cu_seqlens, checkpoints, gate, norm_weight)
        self._args = (ctypes.byref(self.params), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                      _ptr(initial_state), _ptr(cu_seqlens), _ptr(o), _ptr(final_state), _ptr(workspace),
                      ctypes.c_size_t(workspace.numel()), _stream(stream))
        self._lib = load()

    def run(self):
        if self.options is not None:
            _check("kda_chunk_fwd_ex", self._lib.kda_chunk_fwd_ex(self._args[0], ctypes.byref(self.options),
                                                                  *self._args[1:]))
        else:
            _check("kda_chunk_fwd", self._lib.kda_chunk_fwd(*self._args))
        return self.o, self.final_state

    def status(self) -> int:
        """kda_chunk_fwd_status of the last run (synchronises the stream): 0, or KDA_ERR_RANGE;
        raises KdaError for any other status (KDA_ERR_INVALID_ARG: cu_seqlens broke its layout)."""
        st = self._lib.kda_chunk_fwd_status(self._args[10], self._args[12])
        if st not in (0, KDA_ERR_RANGE):
            _check("kda_chunk_fwd_status", st)
        return st

    def check_range(self):
        """Raise KdaError if the last run wrote a value that is not finite (KDA_ERR_RANGE)
        or its cu_seqlens broke the layout (KDA_ERR_INVALID_ARG)."""
        _check("kda_chunk_fwd_status", self.status())

    def _plain_phase(self, name):
        # kda_chunk_fwd_intra / _inter are the two halves of the plain call: they
        # take no options, so a call with options (a per-token alpha, a gate,
        # checkpoints ...) would run with its tensors read in the plain layout
        if self.options is not None:
            raise ValueError(f"{name}: the split phases run the plain call only; this call has options")
        return getattr(self._lib, name)

    def intra(self):
        _check("kda_chunk_fwd_intra", self._plain_phase("kda_chunk_fwd_intra")(*self._args))

    def inter(self):
        _check("kda_chunk_fwd_inter", self._plain_phase("kda_chunk_fwd_inter")(*self._args))
        return self.o, self.final_state


def chunk_fwd(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, chunk_size: int = 64,
              scale: float = 1.0, output_final_state: bool = True, o=None, final_state=None,
              workspace=None, stream=None, o_dtype: Optional[torch.dtype] = None,
              checkpoints=None, ckpt_every: int = 0, decay_floor: float = 0.0, alpha_scalar: bool = False,
              fuse_inputs: bool = False, gate=None, norm_weight=None, norm_eps: float = 0.0,
              check_range: bool = True):
    """Chunked KDA prefill through kda_chunk_fwd.  Returns (o, final_state or None).

    q, k [B,T,H,dk], v [B,T,H,dv] (bf16 or fp32, same dtype), alpha [B,T,H,dk] fp32,
    beta [B,T,H] fp32, initial_state [N,H,dk,dv] fp32 or None, cu_seqlens int32 [N+1] or
    None (device tensors).  ``final_state`` may be ``initial_state`` (in-place resume).
    ``o_dtype`` (default: the dtype of q) is bf16 or fp32.  With ``ckpt_every`` (a
    multiple of 64) the call goes through kda_chunk_fwd_ex and writes the state after
    every ``ckpt_every`` tokens of each sequence into ``checkpoints`` [N,max_ckpts,H,dk,dv].
    ``decay_floor``, ``alpha_scalar`` (alpha [B,T,H]), ``fuse_inputs`` (L2 norm of q, k;
    alpha, beta given as logits) and ``gate`` [B,T,H,dv] with ``norm_weight`` [dv] and
    ``norm_eps`` (output norm and sigmoid gate) are the other kda_chunk_options_t fields.
    With ``check_range`` (the default) the call then reads kda_chunk_fwd_status, which
    synchronises the stream, and raises KdaError (status KDA_ERR_INVALID_ARG) when the device
    found cu_seqlens malformed, or (status KDA_ERR_RANGE) when a written
    value is not finite (an intermediate left the fp16 operand range of the bf16 path).
    """
    pre = Prefill(q, k, v, alpha, beta, initial_state, cu_seqlens, chunk_size, scale,
                  output_final_state, o, final_state, workspace, stream, o_dtype,
                  checkpoints, ckpt_every, decay_floor, alpha_scalar, fuse_inputs, gate, norm_weight,
                  norm_eps)
    out = pre.run()
    if check_range:
        pre.check_range()
    return out


def chunk_fwd_noalloc(q, k, v, alpha, beta, initial_state=None, cu_seqlens=None, o=None, final_state=None,
                      chunk_size: int = 64, scale: float = 1.0, o_dtype: Optional[torch.dtype] = None,
                      stream=None):
    """kda_chunk_fwd_noalloc: kda_chunk_fwd on the library-held scratch, with no workspace.

    The library allocates nothing for the call; ``o`` and ``final_state`` are
    allocated here only when not given (pass both to allocate nothing at all).
    Shapes and dtypes as chunk_fwd.  Returns (o, final_state).
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(k.shape == q.shape and alpha.shape == q.shape, "q, k, alpha must share [B,T,H,dk]")
    _need(v.shape == (B, T, H, dv) and beta.shape == (B, T, H), "v/beta shapes")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    _need(alpha.dtype == torch.float32 and beta.dtype == torch.float32, "alpha, beta must be fp32")
    for t in (q, k, v, alpha, beta):
        _need(_on_device(t) and t.is_contiguous(), "inputs must be contiguous device tensors")
    if cu_seqlens is not None:
        _need(cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2, "cu_seqlens must be int32 [N+1] with N >= 1")
        _dense(cu_seqlens, (cu_seqlens.numel(),), torch.int32, "cu_seqlens")
    n = B if cu_seqlens is None else cu_seqlens.numel() - 1
    _dense(initial_state, (n, H, dk, dv), torch.float32, "initial_state")
    _dense(final_state, (n, H, dk, dv), torch.float32, "final_state")
    o_dtype = q.dtype if o_dtype is None else o_dtype
    _dense(o, v.shape, o_dtype, "o")
    if o is None:
        o = torch.empty(v.shape, dtype=o_dtype, device=v.device)
    if final_state is None:
        final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device)
    params = chunk_params(q, v, cu_seqlens, chunk_size, scale, o_dtype)
    _check("kda_chunk_fwd_noalloc",
           load().kda_chunk_fwd_noalloc(ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                        _ptr(initial_state), _ptr(cu_seqlens), _ptr(o), _ptr(final_state),
                                        _stream(stream)))
    return o, final_state


def chunk_fwd_windowed(q, k, v, alpha, beta, workspace, initial_state=None, cu_seqlens=None, o=None,
                       final_state=None, chunk_size: int = 64, scale: float = 1.0,
                       o_dtype: Optional[torch.dtype] = None, stream=None, check_range: bool = True,
                       cu_seqlens_host=None, checkpoints=None, ckpt_every: int = 0, decay_floor: float = 0.0,
                       alpha_scalar: bool = False, fuse_inputs: bool = False, gate=None, norm_weight=None,
                       norm_eps: float = 0.0):
    """kda_chunk_fwd_windowed(_ex): kda_chunk_fwd(_ex) in the memory of ``workspace`` (a
    256-byte aligned device buffer of any size that holds one chunk's call, or one
    of ``ckpt_every`` tokens with checkpoints).

    Shapes, dtypes and the options (``checkpoints`` ... ``norm_eps``) as chunk_fwd;
    with any option set the call goes through kda_chunk_fwd_windowed_ex.  The
    library plans the windows from a host copy of ``cu_seqlens``:
    ``cu_seqlens_host`` (a CPU int32 tensor with the same values) when given,
    else one made here (the copy synchronises).  ``final_state`` is allocated
    when not given.  Returns (o, final_state).
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(k.shape == q.shape, "q and k must share [B,T,H,dk]")
    _need(alpha.shape == ((B, T, H) if alpha_scalar else q.shape),
          "alpha must be [B,T,H,dk] ([B,T,H] with alpha_scalar)")
    _need(v.shape == (B, T, H, dv) and beta.shape == (B, T, H), "v/beta shapes")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    _need(alpha.dtype == torch.float32 and beta.dtype == torch.float32, "alpha, beta must be fp32")
    for t in (q, k, v, alpha, beta):
        _need(_on_device(t) and t.is_contiguous(), "inputs must be contiguous device tensors")
    _need(isinstance(workspace, torch.Tensor) and _on_device(workspace) and workspace.is_contiguous(),
          "workspace must be a contiguous device tensor")
    cu_host = None
    if cu_seqlens is not None:
        _need(cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2, "cu_seqlens must be int32 [N+1] with N >= 1")
        _dense(cu_seqlens, (cu_seqlens.numel(),), torch.int32, "cu_seqlens")
        if cu_seqlens_host is None:
            cu_host = cu_seqlens.cpu()
        else:
            _need(isinstance(cu_seqlens_host, torch.Tensor) and cu_seqlens_host.device.type == "cpu" and
                  cu_seqlens_host.dtype == torch.int32 and cu_seqlens_host.is_contiguous() and
                  cu_seqlens_host.shape == cu_seqlens.shape, "cu_seqlens_host must be a CPU int32 copy of cu_seqlens")
            cu_host = cu_seqlens_host
    else:
        _need(cu_seqlens_host is None, "cu_seqlens_host must come with cu_seqlens")
    n = B if cu_seqlens is None else cu_seqlens.numel() - 1
    _dense(initial_state, (n, H, dk, dv), torch.float32, "initial_state")
    _dense(final_state, (n, H, dk, dv), torch.float32, "final_state")
    o_dtype = q.dtype if o_dtype is None else o_dtype
    _dense(o, v.shape, o_dtype, "o")
    _check_options(q, v, n, checkpoints, ckpt_every, gate, norm_weight)
    if o is None:
        o = torch.empty(v.shape, dtype=o_dtype, device=v.device)
    if final_state is None:
        final_state = torch.empty((n, H, dk, dv), dtype=torch.float32, device=q.device)
    params = chunk_params(q, v, cu_seqlens, chunk_size, scale, o_dtype)
    options = _chunk_options(checkpoints, ckpt_every, decay_floor, alpha_scalar, fuse_inputs, gate, norm_weight,
                             norm_eps)
    lib = load()
    rest = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state), _ptr(cu_seqlens),
            None if cu_host is None else cu_host.data_ptr(), _ptr(o), _ptr(final_state), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if options is None:
        _check("kda_chunk_fwd_windowed", lib.kda_chunk_fwd_windowed(ctypes.byref(params), *rest))
    else:
        _check("kda_chunk_fwd_windowed_ex",
               lib.kda_chunk_fwd_windowed_ex(ctypes.byref(params), ctypes.byref(options), *rest))
    if check_range:
        _check("kda_chunk_fwd_status", lib.kda_chunk_fwd_status(_ptr(workspace), _stream(stream)))
    return o, final_state


def decode_step(q, k, v, alpha, beta, state, scale: float = 1.0, o=None, stream=None,
                o_dtype: Optional[torch.dtype] = None, state_slots=None, decay_floor: float = 0.0,
                alpha_scalar: bool = False, fuse_inputs: bool = False, gate=None, norm_weight=None,
                norm_eps: float = 0.0, pool_entries: Optional[int] = None):
    """One decode step through kda_decode_step (or kda_decode_step_ex with any option).

    q, k [N,H,dk], alpha [N,H,dk] ([N,H] with ``alpha_scalar``), v [N,H,dv], beta [N,H];
    ``state`` [N,H,dk,dv] is updated in place, or with ``state_slots`` (int32 [N] device)
    it is a pool [P,H,dk,dv] and sequence n updates entry state_slots[n]; a slot outside
    [0, pool_entries) (default P) is skipped on the device and gives o = NaN.  Options as in
    include/kda.h: ``decay_floor``, ``fuse_inputs`` (L2 norm of q, k; alpha, beta logits),
    ``gate`` [N,H,dv] logits with ``norm_weight`` [dv] and ``norm_eps``.
    Returns o [N,H,dv] (``o_dtype``, default the dtype of q).
    """
    N, H, dk = q.shape
    dv = v.shape[-1]
    a_shape = (N, H) if alpha_scalar else (N, H, dk)
    _need(k.shape == q.shape and alpha.shape == a_shape and v.shape == (N, H, dv)
          and beta.shape == (N, H), "decode shapes")
    if state_slots is None:
        _need(state.shape == (N, H, dk, dv), "state must be [N,H,dk,dv]")
    else:
        _need(state.dim() == 4 and state.shape[1:] == (H, dk, dv), "state pool must be [P,H,dk,dv]")
        _dense(state_slots, (N,), torch.int32, "state_slots")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    _need(alpha.dtype == torch.float32 and beta.dtype == torch.float32
          and state.dtype == torch.float32, "alpha, beta, state must be fp32")
    for t in (q, k, v, alpha, beta):
        _need(_on_device(t) and t.is_contiguous(), "inputs must be contiguous device tensors")
    _dense(state, state.shape, torch.float32, "state")
    _dense(gate, v.shape, q.dtype, "gate")
    _dense(norm_weight, (dv,), torch.float32, "norm_weight")
    o_dtype = q.dtype if o_dtype is None else o_dtype
    _dense(o, v.shape, o_dtype, "o")
    if o is None:
        o = torch.empty(v.shape, dtype=o_dtype, device=v.device)
    lib = load()
    head = (N, H, dk, dv, float(scale), _code(q.dtype), _code(o_dtype))
    tail = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(o), _stream(stream))
    if (state_slots is None and not decay_floor and not alpha_scalar and not fuse_inputs and gate is None
            and norm_weight is None):
        _check("kda_decode_step", lib.kda_decode_step(*head, *tail))
    else:
        if state_slots is not None:
            pool_entries = state.shape[0] if pool_entries is None else int(pool_entries)
            _need(0 < pool_entries <= state.shape[0], "pool_entries must lie in [1, P]")
        opt = DecodeOptions(state_slots=None if state_slots is None else state_slots.data_ptr(),
                            pool_entries=0 if state_slots is None else pool_entries,
                            decay_floor=float(decay_floor), alpha_mode=int(bool(alpha_scalar)),
                            fuse_inputs=int(bool(fuse_inputs)), gate=None if gate is None else gate.data_ptr(),
                            norm_weight=None if norm_weight is None else norm_weight.data_ptr(),
                            norm_eps=float(norm_eps))
        _check("kda_decode_step_ex", lib.kda_decode_step_ex(*head, ctypes.byref(opt), *tail))
    return o
