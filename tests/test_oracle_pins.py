"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test fixes the oracle to something independent of its code: a hand-worked
example, a closed form, a special case that reduces to a textbook routine, or
a brute-force expansion written differently (explicit transition matrices).
Together they fail on a dropped term, a wrong sign, a swapped index or a
transposed operand anywhere in the recurrence:

* recall on the pre-decay state           -> exact recall (P4), worked example
* read before the correction              -> exact recall, alpha = 0 closed form
* decay on value channels instead of keys -> pure-decay closed form with dk != dv
* beta on the write only (not the erase)  -> scalar closed form, slot EMA
* q / k swapped, head or token mis-index  -> plain GEMM case, multi-head cases
"""
import os

import numpy as np
import pytest
import torch

from oracle import kda_oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kda_worked_example.txt")


def _rand_inputs(B, T, H, dk, dv, seed, dtype=torch.float64, unit_keys=True, alpha=None,
                 beta=None, s0=True, N=None):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, T, H, dk, generator=g, dtype=torch.float64)
    k = torch.randn(B, T, H, dk, generator=g, dtype=torch.float64)
    if unit_keys:
        k = k / k.norm(dim=-1, keepdim=True)
        q = q / q.norm(dim=-1, keepdim=True)
    v = torch.randn(B, T, H, dv, generator=g, dtype=torch.float64)
    a = torch.sigmoid(torch.randn(B, T, H, dk, generator=g, dtype=torch.float64) + 2.0)
    b = torch.sigmoid(torch.randn(B, T, H, generator=g, dtype=torch.float64))
    if alpha is not None:
        a = torch.full_like(a, alpha)
    if beta is not None:
        b = torch.full_like(b, beta)
    n = B if N is None else N
    S0 = torch.randn(n, H, dk, dv, generator=g, dtype=torch.float64) if s0 else None
    return [x.to(dtype) if x is not None else None for x in (q, k, v)] + [a, b, S0]


def _np(x):
    return x.to(torch.float64).numpy()


def test_worked_example_golden():
    """Hand-derived two-token example (tests/golden/kda_worked_example.txt)."""
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, *nums = line.split()
            vals[name] = np.array([float(x) for x in nums])
    S0 = torch.tensor(vals["S0"]).reshape(1, 1, 2, 2)
    alpha = torch.tensor(vals["alpha"]).reshape(1, 2, 1, 2)
    beta = torch.tensor(vals["beta"]).reshape(1, 2, 1)
    k = torch.tensor(vals["k"]).reshape(1, 2, 1, 2)
    v = torch.tensor(vals["v"]).reshape(1, 2, 1, 2)
    q = torch.tensor(vals["q"]).reshape(1, 2, 1, 2)
    o, S = kda_oracle.forward(q, k, v, alpha, beta, S0=S0)
    np.testing.assert_allclose(o.reshape(-1), vals["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S.reshape(-1), vals["S_final"], rtol=0, atol=1e-14)


def test_p1_identity_gate_is_plain_gemm():
    """alpha = 1, beta = 0: the state never changes and o_t = scale * S0^T q_t."""
    q, k, v, a, b, S0 = _rand_inputs(2, 9, 3, 5, 7, seed=1, alpha=1.0, beta=0.0)
    o, S = kda_oracle.forward(q, k, v, a, b, S0=S0, scale=0.37)
    np.testing.assert_array_equal(S, _np(S0))
    ref = 0.37 * np.einsum("bthc,bhcj->bthj", _np(q), _np(S0))
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-13)


def test_p2_zero_decay_forgets_everything():
    """alpha = 0: S_t = beta_t k_t v_t^T and o_t = beta_t (q_t . k_t) v_t."""
    q, k, v, a, b, S0 = _rand_inputs(1, 6, 2, 4, 3, seed=2, alpha=0.0, unit_keys=False)
    o, S = kda_oracle.forward(q, k, v, a, b, S0=S0)
    qn, kn, vn, bn = _np(q), _np(k), _np(v), _np(b)
    ref_S = bn[0, -1][:, None, None] * kn[0, -1][:, :, None] * vn[0, -1][:, None, :]
    np.testing.assert_allclose(S[0], ref_S, rtol=1e-13, atol=1e-13)
    ref_o = (bn[..., None] * np.sum(qn * kn, -1, keepdims=True)) * vn
    np.testing.assert_allclose(o, ref_o, rtol=1e-13, atol=1e-13)


def test_p3_pure_decay_closed_form():
    """beta = 0: S_t = diag(prod_{s<=t} alpha_s) S0; o_t = S0^T (gamma_t * q_t).  dk != dv."""
    q, k, v, a, b, S0 = _rand_inputs(1, 11, 2, 6, 3, seed=3, beta=0.0)
    o, S = kda_oracle.forward(q, k, v, a, b, S0=S0)
    gam = np.cumprod(_np(a)[0], axis=0)                      # [T, H, dk]
    ref_S = gam[-1][:, :, None] * _np(S0)[0]
    np.testing.assert_allclose(S[0], ref_S, rtol=1e-13, atol=1e-14)
    ref_o = np.einsum("thc,hcj->thj", gam * _np(q)[0], _np(S0)[0])
    np.testing.assert_allclose(o[0], ref_o, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", [4, 5])
def test_p4_exact_associative_recall(seed):
    """Unit keys, beta = 1, q = k: o_t = v_t exactly, for any decay and any state.

    Holds only if the recall uses the decayed state and the read follows the
    correction.
    """
    q, k, v, a, b, S0 = _rand_inputs(1, 13, 2, 8, 5, seed=seed, beta=1.0)
    o, _ = kda_oracle.forward(k, k, v, a, b, S0=S0)
    np.testing.assert_allclose(o, _np(v), rtol=0, atol=1e-12)


def test_p5_standard_basis_keys_slot_ema():
    """Keys e_{i_t}: each key row is an independent slot with an exponential moving average.

    slot c decays by alpha_t[c] every token; the addressed slot then moves a
    beta share towards v_t.  A query e_j reads slot j.
    """
    rng = np.random.default_rng(6)
    T, dk, dv = 20, 4, 3
    idx = rng.integers(0, dk, size=T)
    k = np.zeros((1, T, 1, dk)); k[0, np.arange(T), 0, idx] = 1.0
    qidx = rng.integers(0, dk, size=T)
    q = np.zeros((1, T, 1, dk)); q[0, np.arange(T), 0, qidx] = 1.0
    v = rng.standard_normal((1, T, 1, dv))
    a = rng.uniform(0.3, 1.0, size=(1, T, 1, dk))
    b = rng.uniform(0.0, 1.0, size=(1, T, 1))
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, S = kda_oracle.forward(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                              torch.from_numpy(a), torch.from_numpy(b), S0=torch.from_numpy(S0))
    slots = S0[0, 0].copy()
    for t in range(T):
        slots *= a[0, t, 0][:, None]
        i = idx[t]
        slots[i] = (1.0 - b[0, t, 0]) * slots[i] + b[0, t, 0] * v[0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], slots[qidx[t]], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S[0, 0], slots, rtol=1e-13, atol=1e-13)
    # alpha = beta = 1: a query on slot i returns the last value written there
    a1 = np.ones_like(a); b1 = np.ones_like(b)
    o1, _ = kda_oracle.forward(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                               torch.from_numpy(a1), torch.from_numpy(b1))
    for t in range(T):
        written = [s for s in range(t + 1) if idx[s] == qidx[t]]
        want = v[0, written[-1], 0] if written else np.zeros(dv)
        np.testing.assert_allclose(o1[0, t, 0], want, rtol=0, atol=1e-14)


def test_p6_scalar_geometric_closed_form():
    """d = 1, alpha = a, beta = b, k = v = q = 1, s0 = 0: s_t = b (1 - r^t) / (1 - r), r = (1-b) a."""
    T, av, bv = 40, 0.9, 0.3
    ones = torch.ones(1, T, 1, 1, dtype=torch.float64)
    o, S = kda_oracle.forward(ones, ones, ones, ones * av, torch.full((1, T, 1), bv,
                              dtype=torch.float64))
    r = (1 - bv) * av
    t = np.arange(1, T + 1)
    np.testing.assert_allclose(o[0, :, 0, 0], bv * (1 - r ** t) / (1 - r), rtol=1e-13)
    np.testing.assert_allclose(S[0, 0, 0, 0], bv * (1 - r ** T) / (1 - r), rtol=1e-13)


def _brute_force(q, k, v, a, b, S0):
    """S_t = Phi_{t,0} S0 + sum_{s<=t} Phi_{t,s} beta_s k_s v_s^T with
    A_s = (I - beta_s k_s k_s^T) diag(alpha_s) and Phi_{t,s} = A_t ... A_{s+1}."""
    T, dk = k.shape[0], k.shape[1]
    A = [(np.eye(dk) - b[s] * np.outer(k[s], k[s])) @ np.diag(a[s]) for s in range(T)]

    def phi(t, s):  # product A_t A_{t-1} ... A_{s+1} (tokens numbered from 1)
        m = np.eye(dk)
        for u in range(s + 1, t + 1):
            m = A[u - 1] @ m
        return m

    outs, St = [], None
    for t in range(1, T + 1):
        St = phi(t, 0) @ S0
        for s in range(1, t + 1):
            St = St + phi(t, s) @ (b[s - 1] * np.outer(k[s - 1], v[s - 1]))
        outs.append(St.T @ q[t - 1])
    return np.array(outs), St


@pytest.mark.parametrize("T,dk,dv,seed", [(1, 3, 2, 7), (5, 4, 6, 8), (8, 16, 5, 9), (8, 16, 16, 10)])
def test_p7_brute_force_expansion(T, dk, dv, seed):
    q, k, v, a, b, S0 = _rand_inputs(1, T, 2, dk, dv, seed=seed, unit_keys=(seed % 2 == 0))
    o, S = kda_oracle.forward(q, k, v, a, b, S0=S0)
    for h in range(2):
        ref_o, ref_S = _brute_force(_np(q)[0, :, h], _np(k)[0, :, h], _np(v)[0, :, h],
                                    _np(a)[0, :, h], _np(b)[0, :, h], _np(S0)[0, h])
        np.testing.assert_allclose(o[0, :, h], ref_o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(S[0, h], ref_S, rtol=1e-11, atol=1e-12)


def test_p8_linearity_in_values_and_state():
    q, k, v1, a, b, S01 = _rand_inputs(1, 12, 2, 6, 4, seed=11)
    _, _, v2, _, _, S02 = _rand_inputs(1, 12, 2, 6, 4, seed=12)
    c = -1.7
    o1, s1 = kda_oracle.forward(q, k, v1, a, b, S0=S01)
    o2, s2 = kda_oracle.forward(q, k, v2, a, b, S0=S02)
    o3, s3 = kda_oracle.forward(q, k, v1 + c * v2, a, b, S0=S01 + c * S02)
    np.testing.assert_allclose(o3, o1 + c * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s3, s1 + c * s2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("split", [1, 7, 19])
def test_p8_resume_from_a_checkpoint(split):
    """Running a prefix, then the rest from the prefix's final state, equals the full run."""
    q, k, v, a, b, S0 = _rand_inputs(1, 20, 3, 5, 6, seed=13)
    o, S = kda_oracle.forward(q, k, v, a, b, S0=S0)
    sl1, sl2 = slice(0, split), slice(split, 20)
    oa, Sa = kda_oracle.forward(q[:, sl1], k[:, sl1], v[:, sl1], a[:, sl1], b[:, sl1], S0=S0)
    ob, Sb = kda_oracle.forward(q[:, sl2], k[:, sl2], v[:, sl2], a[:, sl2], b[:, sl2],
                                S0=torch.from_numpy(Sa))
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Sb, S, rtol=1e-13, atol=1e-13)


def test_p8_packed_equals_separate_runs_and_head_subset():
    lens = [5, 0, 9, 1, 4]
    T = sum(lens)
    q, k, v, a, b, S0 = _rand_inputs(1, T, 3, 4, 5, seed=14, N=len(lens))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, S = kda_oracle.forward(q, k, v, a, b, S0=S0, cu_seqlens=cu)
    for n, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        if e == s:
            np.testing.assert_array_equal(S[n], _np(S0)[n])  # empty sequence: final = initial
            continue
        on, Sn = kda_oracle.forward(q[:, s:e], k[:, s:e], v[:, s:e], a[:, s:e], b[:, s:e],
                                    S0=S0[n:n + 1])
        np.testing.assert_allclose(o[:, s:e], on, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(S[n], Sn[0], rtol=1e-13, atol=1e-13)
    oh, Sh = kda_oracle.forward(q, k, v, a, b, S0=S0, cu_seqlens=cu, heads=(1, 3))
    np.testing.assert_array_equal(oh, o[:, :, 1:3])
    np.testing.assert_array_equal(Sh, S[:, 1:3])


def test_stored_dtypes_are_read_exactly():
    """bf16 and fp32 inputs equal their exact fp64 upcasts."""
    q, k, v, a, b, S0 = _rand_inputs(2, 7, 2, 8, 8, seed=15)
    qb, kb, vb = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    o1, s1 = kda_oracle.forward(qb, kb, vb, a.float(), b.float(), S0=S0.float())
    o2, s2 = kda_oracle.forward(qb.double(), kb.double(), vb.double(), a.float().double(),
                                b.float().double(), S0=S0.float().double())
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_decode_wrapper_matches_forward():
    """The step-major decode wrapper is the same recurrence as a packed forward."""
    steps, N, H, d = 6, 3, 2, 4
    q, k, v, a, b, S0 = _rand_inputs(steps, N, H, d, d, seed=16, N=N)
    o, S = kda_oracle.decode(S0, q, k, v, a, b)
    for n in range(N):
        on, Sn = kda_oracle.forward(q[:, n][None], k[:, n][None], v[:, n][None], a[:, n][None],
                                    b[:, n][None], S0=S0[n:n + 1])
        np.testing.assert_allclose(o[:, n], on[0], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(S[n], Sn[0], rtol=1e-13, atol=1e-13)
