"""ctypes binding of the fp64 CPU oracle (test infrastructure only).

The recurrence itself lives in kda_oracle.c; this file only marshals tensors.
Inputs are taken exactly as stored (bf16 / fp32 / fp64) and upcast inside the
oracle; outputs are fp64 numpy arrays.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import build as _build

_F32, _BF16, _F64 = 0, 1, 2
_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        fn = lib.kda_oracle_forward
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                       ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                       ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        fx = lib.kda_oracle_forward_ex
        fx.restype = ctypes.c_int
        fx.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                       ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                       ctypes.c_void_p, ctypes.c_int32,
                       ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                       ctypes.c_double, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double,
                       ctypes.c_void_p, ctypes.c_void_p]
        lib.kda_oracle_threads.restype = ctypes.c_int
        lib.kda_oracle_threads.argtypes = []
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle runs with."""
    return int(_load().kda_oracle_threads())


def _as_cpu(x):
    """(contiguous CPU tensor kept alive, pointer, dtype code)."""
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    x = x.detach().to("cpu").contiguous()
    if x.dtype == torch.bfloat16:
        return x, x.view(torch.int16).data_ptr(), _BF16
    if x.dtype == torch.float32:
        return x, x.data_ptr(), _F32
    if x.dtype == torch.float64:
        return x, x.data_ptr(), _F64
    raise TypeError(f"oracle: unsupported dtype {x.dtype}")


def forward(q, k, v, alpha, beta, S0=None, cu_seqlens=None, scale: float = 1.0,
            heads: Optional[Sequence[int]] = None, ckpt_every: int = 0, max_ckpts: int = 0,
            decay_floor: float = 0.0, alpha_scalar: bool = False, fuse_inputs: bool = False,
            gate=None, norm_weight=None, norm_eps: float = 0.0, return_ckpt: bool = False):
    """Token-by-token fp64 KDA over q,k [B,T,H,dk], v [B,T,H,dv], alpha [B,T,H,dk], beta [B,T,H].

    Without ``cu_seqlens`` each of the B rows is one sequence; with it B must be
    1 and sequence n covers tokens [cu[n], cu[n+1]).  ``S0`` is [N,H,dk,dv] or
    None (zeros).  ``heads`` = (h_begin, h_end) restricts the computed heads.
    Options (kda_oracle.c documents each with its source): ``ckpt_every`` /
    ``max_ckpts`` state checkpoints, ``decay_floor``, ``alpha_scalar`` (alpha
    [B,T,H]), ``fuse_inputs`` (L2 norm of q, k; sigmoid of alpha, beta logits),
    ``gate`` [B,T,H,dv] with ``norm_weight`` [dv] and ``norm_eps`` (output norm
    and sigmoid gate).
    Returns (o [B,T,nh,dv], S_final [N,nh,dk,dv]) as float64 numpy arrays, and
    the checkpoints [N,max_ckpts,nh,dk,dv] (NaN where not reached) when
    ``return_ckpt``.
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        assert B == 1
        cu = np.asarray(torch.as_tensor(cu_seqlens).cpu().numpy(), dtype=np.int64)
    n = len(cu) - 1
    h0, h1 = (0, H) if heads is None else (int(heads[0]), int(heads[1]))
    nh = h1 - h0
    keep = []
    qt, qp, qd = _as_cpu(q)
    kt, kp, kd = _as_cpu(k)
    vt, vp, vd = _as_cpu(v)
    if not (qd == kd == vd):
        raise TypeError("oracle: q, k, v must share a dtype")
    at, ap, ad = _as_cpu(alpha)
    bt, bp, bd = _as_cpu(beta)
    keep += [qt, kt, vt, at, bt]
    sp, sd = None, _F32
    if S0 is not None:
        st, sp, sd = _as_cpu(S0)
        keep.append(st)
    gp, gd = None, _F32
    if gate is not None:
        gt, gp, gd = _as_cpu(gate)
        keep.append(gt)
    wp = None
    if norm_weight is not None:
        wt = torch.as_tensor(norm_weight).detach().to("cpu", torch.float32).contiguous()
        keep.append(wt)
        wp = wt.data_ptr()
    o = np.zeros((B * T, nh, dv), dtype=np.float64)
    s_fin = np.zeros((n, nh, dk, dv), dtype=np.float64)
    ck = np.full((n, max(max_ckpts, 1), nh, dk, dv), np.nan) if ckpt_every > 0 else None
    cu_c = np.ascontiguousarray(cu)
    rc = _load().kda_oracle_forward_ex(n, cu_c.ctypes.data, H, dk, dv, h0, h1, float(scale),
                                       qp, kp, vp, qd, ap, ad, bp, bd, sp, sd,
                                       int(ckpt_every), int(max_ckpts),
                                       None if ck is None else ck.ctypes.data,
                                       float(decay_floor), int(bool(alpha_scalar)), int(bool(fuse_inputs)),
                                       gp, gd, wp, float(norm_eps),
                                       o.ctypes.data, s_fin.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward_ex failed with code {rc}")
    if return_ckpt:
        return o.reshape(B, T, nh, dv), s_fin, ck
    return o.reshape(B, T, nh, dv), s_fin


def decode(S0, q, k, v, alpha, beta, scale: float = 1.0, heads=None, state_slots=None, **options):
    """Run ``steps`` successive single-token steps of N sequences.

    q,k,alpha [steps,N,H,dk] (alpha [steps,N,H] with ``alpha_scalar``), v [steps,N,H,dv],
    beta [steps,N,H], S0 [N,H,dk,dv]; with ``state_slots`` (N slot indices) S0 is a
    pool [P,H,dk,dv] and sequence n starts from pool slot state_slots[n] (the
    paged state pool of "Kimi K3 architecture: KDA, MLA and MoE", section
    "Serving K3 means managing two cache lifecycles").  The oracle treats each
    sequence's steps as its tokens in order, which is the recurrence applied
    one token at a time; ``options`` are those of ``forward`` (gate
    [steps,N,H,dv]).  Returns (o [steps,N,nh,dv], S_final [N,nh,dk,dv]).
    """
    steps, N = q.shape[0], q.shape[1]

    def tm(x):  # [steps, N, ...] -> [1, N*steps, ...] with each sequence contiguous
        x = torch.as_tensor(x)
        return x.transpose(0, 1).contiguous().reshape(1, N * steps, *x.shape[2:])

    if state_slots is not None:
        S0 = torch.as_tensor(S0)[torch.as_tensor(state_slots, dtype=torch.long)]
    if options.get("gate") is not None:
        options = dict(options, gate=tm(options["gate"]))
    cu = np.arange(N + 1, dtype=np.int64) * steps
    o, s = forward(tm(q), tm(k), tm(v), tm(alpha), tm(beta), S0=S0, cu_seqlens=cu,
                   scale=scale, heads=heads, **options)
    o = o.reshape(N, steps, o.shape[2], o.shape[3]).transpose(1, 0, 2, 3)
    return np.ascontiguousarray(o), s
