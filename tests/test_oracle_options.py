"""Pins of the oracle's options: state checkpoints, decay floor, scalar gate,
fused input transforms and the output norm + gate.

Each pin ties an option to something other than the option's own code: the
plain recurrence on a truncated or transformed input (computed with numpy /
scipy), closed forms, or invariants that a plausible mistake breaks.
"""
import numpy as np
import pytest
import torch
from scipy.special import expit

from oracle import kda_oracle

RTOL = 1e-12


def _inputs(B=1, T=24, H=2, dk=8, dv=6, seed=0, lengths=None):
    g = torch.Generator().manual_seed(seed)
    tot = B * T if lengths is None else sum(lengths)
    shape_t = (B, T) if lengths is None else (1, tot)
    q = torch.randn(*shape_t, H, dk, generator=g, dtype=torch.float64)
    k = torch.nn.functional.normalize(torch.randn(*shape_t, H, dk, generator=g, dtype=torch.float64), dim=-1)
    v = torch.randn(*shape_t, H, dv, generator=g, dtype=torch.float64)
    alpha = torch.sigmoid(torch.randn(*shape_t, H, dk, generator=g, dtype=torch.float64) + 2.0)
    beta = torch.sigmoid(torch.randn(*shape_t, H, generator=g, dtype=torch.float64))
    n = B if lengths is None else len(lengths)
    s0 = 0.1 * torch.randn(n, H, dk, dv, generator=g, dtype=torch.float64)
    cu = None if lengths is None else torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64)
    return q, k, v, alpha, beta, s0, cu


def _close(a, b, tol=RTOL):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))))
    assert np.max(np.abs(a - b)) <= tol * scale, np.max(np.abs(a - b))


# --- state checkpoints --------------------------------------------------------------------------

def test_checkpoints_equal_states_of_truncated_prefixes():
    lengths = [5, 12, 0, 8, 16]
    every, mx = 4, 3
    q, k, v, alpha, beta, s0, cu = _inputs(lengths=lengths, seed=1)
    o, s, ck = kda_oracle.forward(q, k, v, alpha, beta, S0=s0, cu_seqlens=cu, ckpt_every=every,
                                  max_ckpts=mx, return_ckpt=True)
    for n, L in enumerate(lengths):
        a = int(cu[n])
        for j in range(mx):
            end = (j + 1) * every
            if end > L:
                assert np.all(np.isnan(ck[n, j])), (n, j)   # not reached: left untouched
                continue
            sl = slice(a, a + end)
            _, s_pref = kda_oracle.forward(q[:, sl], k[:, sl], v[:, sl], alpha[:, sl], beta[:, sl],
                                           S0=s0[n:n + 1])
            _close(ck[n, j], s_pref[0])
    # a checkpoint at the end of a sequence is its final state (length 12 = 3 * 4; length 8 = 2 * 4)
    _close(ck[1, 2], s[1])
    _close(ck[3, 1], s[3])


def test_checkpoints_resume():
    q, k, v, alpha, beta, s0, _ = _inputs(B=1, T=20, seed=2)
    o, s, ck = kda_oracle.forward(q, k, v, alpha, beta, S0=s0, ckpt_every=8, max_ckpts=2, return_ckpt=True)
    # resuming from checkpoint 1 (token 16) reproduces the tail of the outputs and the final state
    o2, s2 = kda_oracle.forward(q[:, 16:], k[:, 16:], v[:, 16:], alpha[:, 16:], beta[:, 16:],
                                S0=torch.from_numpy(ck[:, 1]))
    _close(o2, o[:, 16:])
    _close(s2, s)


# --- decay floor --------------------------------------------------------------------------------

def test_floor_one_keeps_state_when_beta_zero():
    q, k, v, alpha, beta, s0, _ = _inputs(seed=3)
    o, s = kda_oracle.forward(q, k, v, alpha, torch.zeros_like(beta), S0=s0, decay_floor=1.0)
    _close(s, s0.numpy())
    # o_t = S0^T q_t: a plain contraction
    _close(o[0], np.einsum("thc,hcj->thj", q[0].numpy(), s0[0].numpy()))


def test_floor_raises_only_values_below_it():
    q, k, v, alpha, beta, s0, _ = _inputs(seed=4)
    f = 0.9
    o, s = kda_oracle.forward(q, k, v, alpha, beta, S0=s0, decay_floor=f)
    o_ref, s_ref = kda_oracle.forward(q, k, v, torch.clamp(alpha, min=f), beta, S0=s0)
    _close(o, o_ref)
    _close(s, s_ref)
    lo = float(alpha.min()) * 0.5   # a floor below every alpha changes nothing
    o3, s3 = kda_oracle.forward(q, k, v, alpha, beta, S0=s0, decay_floor=lo)
    o4, s4 = kda_oracle.forward(q, k, v, alpha, beta, S0=s0)
    _close(o3, o4)
    _close(s3, s4)


def test_floor_scalar_closed_form():
    # d = 1, alpha = 0 below the floor f, beta = 0: s_t = f^t s0
    T, f, s0 = 9, 0.8, 1.7
    z = torch.zeros(1, T, 1, 1, dtype=torch.float64)
    q = torch.ones_like(z)
    _, s = kda_oracle.forward(q, z, z, z, torch.zeros(1, T, 1, dtype=torch.float64),
                              S0=torch.full((1, 1, 1, 1), s0, dtype=torch.float64), decay_floor=f)
    assert abs(s[0, 0, 0, 0] - f ** T * s0) < 1e-15


# --- scalar gate --------------------------------------------------------------------------------

def test_scalar_gate_equals_broadcast_channel_gate():
    q, k, v, _, beta, s0, cu = _inputs(lengths=[7, 11], seed=5)
    g = torch.Generator().manual_seed(55)
    a_s = torch.sigmoid(torch.randn(1, 18, 2, generator=g, dtype=torch.float64) + 1.0)
    o, s = kda_oracle.forward(q, k, v, a_s, beta, S0=s0, cu_seqlens=cu, alpha_scalar=True)
    a_c = a_s[..., None].expand(*a_s.shape, q.shape[-1]).contiguous()
    o_ref, s_ref = kda_oracle.forward(q, k, v, a_c, beta, S0=s0, cu_seqlens=cu)
    _close(o, o_ref)
    _close(s, s_ref)


def test_scalar_gate_pure_decay_closed_form():
    q, k, v, _, beta, s0, _ = _inputs(seed=6)
    a_s = torch.sigmoid(torch.randn(1, 24, 2, dtype=torch.float64, generator=torch.Generator().manual_seed(6)))
    o, s = kda_oracle.forward(q, k, v, a_s, torch.zeros_like(beta), S0=s0, alpha_scalar=True)
    prod = a_s[0].prod(dim=0).numpy()                       # [H]
    _close(s[0], prod[:, None, None] * s0[0].numpy())


# --- fused input transforms ---------------------------------------------------------------------

def _logit(p):
    return torch.log(p) - torch.log1p(-p)


def test_fused_inputs_equal_transformed_plain_run():
    q, k, v, alpha, beta, s0, cu = _inputs(lengths=[9, 15], seed=7)
    g = torch.Generator().manual_seed(77)
    qr = 3.0 * torch.randn(q.shape, generator=g, dtype=torch.float64)
    kr = 0.5 * torch.randn(k.shape, generator=g, dtype=torch.float64)
    al = torch.randn(alpha.shape, generator=g, dtype=torch.float64) + 2.0
    bl = torch.randn(beta.shape, generator=g, dtype=torch.float64)
    o, s = kda_oracle.forward(qr, kr, v, al, bl, S0=s0, cu_seqlens=cu, fuse_inputs=True)
    qn = qr.numpy() / np.maximum(np.linalg.norm(qr.numpy(), axis=-1, keepdims=True), 1e-12)
    kn = kr.numpy() / np.maximum(np.linalg.norm(kr.numpy(), axis=-1, keepdims=True), 1e-12)
    o_ref, s_ref = kda_oracle.forward(qn, kn, v, expit(al.numpy()), expit(bl.numpy()), S0=s0, cu_seqlens=cu)
    _close(o, o_ref)
    _close(s, s_ref)


def test_fused_inputs_ignore_positive_rescaling_of_q_and_k():
    q, k, v, alpha, beta, s0, _ = _inputs(seed=8)
    g = torch.Generator().manual_seed(88)
    cq = torch.rand(*q.shape[:-1], 1, generator=g, dtype=torch.float64) * 10 + 0.1
    ck = torch.rand(*k.shape[:-1], 1, generator=g, dtype=torch.float64) * 10 + 0.1
    al, bl = _logit(alpha), _logit(beta)
    o1, s1 = kda_oracle.forward(q, k, v, al, bl, S0=s0, fuse_inputs=True)
    o2, s2 = kda_oracle.forward(q * cq, k * ck, v, al, bl, S0=s0, fuse_inputs=True)
    _close(o1, o2, 1e-11)
    _close(s1, s2, 1e-11)


def test_fused_saturated_logits_reduce_to_closed_forms():
    q, k, v, alpha, beta, s0, _ = _inputs(seed=9)
    big = torch.full_like(alpha, 40.0)            # sigmoid(40) == 1 in fp64
    o, s = kda_oracle.forward(q, k, v, big, torch.full_like(beta, -40.0), S0=s0, fuse_inputs=True)
    # beta ~ 4e-18, alpha == 1: the state stays S0 and o_t = S0^T (q_t / |q_t|)
    qn = q[0].numpy() / np.linalg.norm(q[0].numpy(), axis=-1, keepdims=True)
    _close(s, s0.numpy(), 1e-15)
    _close(o[0], np.einsum("thc,hcj->thj", qn, s0[0].numpy()), 1e-14)


def test_fused_zero_vector_stays_zero():
    q, k, v, alpha, beta, s0, _ = _inputs(seed=10)
    k0 = k.clone()
    k0[:, 3] = 0.0    # token 3 writes nothing: its normalised key is 0
    al, bl = _logit(alpha), _logit(beta)
    o, s = kda_oracle.forward(q, k0, v, al, bl, S0=s0, fuse_inputs=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))


# --- output norm and sigmoid gate ---------------------------------------------------------------

def test_gate_output_rows_have_unit_rms():
    q, k, v, alpha, beta, s0, _ = _inputs(seed=11)
    gate = torch.full_like(v, 40.0)
    o, _ = kda_oracle.forward(q, k, v, alpha, beta, S0=s0, gate=gate, norm_eps=0.0)
    rms = np.sqrt(np.mean(o ** 2, axis=-1))
    _close(rms, np.ones_like(rms), 1e-13)


def test_gate_equals_numpy_epilogue_on_plain_output():
    q, k, v, alpha, beta, s0, cu = _inputs(lengths=[10, 14], seed=12)
    g = torch.Generator().manual_seed(121)
    gate = torch.randn(v.shape, generator=g, dtype=torch.float64)
    w = torch.rand(v.shape[-1], generator=g, dtype=torch.float32) + 0.5
    eps = 1e-5
    o, s = kda_oracle.forward(q, k, v, alpha, beta, S0=s0, cu_seqlens=cu, scale=0.7, gate=gate,
                              norm_weight=w, norm_eps=eps)
    op, sp = kda_oracle.forward(q, k, v, alpha, beta, S0=s0, cu_seqlens=cu, scale=0.7)
    ref = op / np.sqrt(np.mean(op ** 2, axis=-1, keepdims=True) + eps) * w.double().numpy() * expit(gate.numpy())
    _close(o, ref)
    _close(s, sp)                 # the epilogue does not touch the state
    # a zero gate logit halves the output of a saturated gate
    o0, _ = kda_oracle.forward(q, k, v, alpha, beta, S0=s0, cu_seqlens=cu, scale=0.7,
                               gate=torch.zeros_like(gate), norm_weight=w, norm_eps=eps)
    o1, _ = kda_oracle.forward(q, k, v, alpha, beta, S0=s0, cu_seqlens=cu, scale=0.7,
                               gate=torch.full_like(gate, 40.0), norm_weight=w, norm_eps=eps)
    _close(o0, 0.5 * o1)


# --- paged decode -------------------------------------------------------------------------------

def test_decode_state_slots_pick_pool_entries():
    g = torch.Generator().manual_seed(13)
    steps, N, H, dk, dv, P = 3, 3, 2, 8, 4, 5
    q = torch.randn(steps, N, H, dk, generator=g, dtype=torch.float64)
    k = torch.nn.functional.normalize(torch.randn(steps, N, H, dk, generator=g, dtype=torch.float64), dim=-1)
    v = torch.randn(steps, N, H, dv, generator=g, dtype=torch.float64)
    a = torch.sigmoid(torch.randn(steps, N, H, dk, generator=g, dtype=torch.float64))
    b = torch.sigmoid(torch.randn(steps, N, H, generator=g, dtype=torch.float64))
    pool = torch.randn(P, H, dk, dv, generator=g, dtype=torch.float64)
    slots = [4, 0, 2]
    o, s = kda_oracle.decode(pool, q, k, v, a, b, state_slots=slots)
    for n, sl in enumerate(slots):
        o1, s1 = kda_oracle.decode(pool[sl:sl + 1], q[:, n:n + 1], k[:, n:n + 1], v[:, n:n + 1],
                                   a[:, n:n + 1], b[:, n:n + 1])
        _close(o[:, n:n + 1], o1)
        _close(s[n:n + 1], s1)
