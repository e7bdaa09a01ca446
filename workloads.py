"""Seeded synthetic inputs for the KDA token mixer.

This module only draws random numbers and shapes them into the inputs of the
KDA box: it holds none of the recurrence's arithmetic.  The oracle (under
``oracle/``) and the HIP path both take their inputs from here.

Input recipe (the pre-processing the KDA layer applies before its core, per the
KDA inset of Visual 1 on the "Kimi K3 Architecture Teardown" page):

* q, k ~ N(0, 1), then L2-normalised per (token, head) over the key channels;
* v = SiLU(N(0, 1));
* alpha = sigmoid(N(mu, 1)) per key channel (mu = 3, or 4 for slow decay);
* beta  = sigmoid(N(0, 1)), one scalar per (token, head);
* S0 = 0, or N(0, 0.02) (0.02 read as the standard deviation) per
  (sequence, head) where a prefix-cache resume is modelled.

Every draw is made in fp32 on a CPU ``torch.Generator`` seeded with
``20261200 + config index``, in the order q, k, v, alpha, beta, S0.  The packed
workload first draws its lengths from that seed and its tensors from the seed
plus 1000; the decode workload draws its initial states from the seed plus
500.  q, k and v are cast once to their storage dtype
(round to nearest even); alpha, beta and S0 stay fp32.  Large tensors are drawn
in fixed blocks of tokens so that host memory stays bounded; the result is a
deterministic function of the seed and the shape.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

SEED_BASE = 20261200
_BLOCK_TOKENS = 16384


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one KDA call (prefill) or of a run of decode steps."""

    name: str
    index: int
    batch: int                 # B (1 when packed)
    seqlen: int                # T per row (prefill) ; 1 for decode
    heads: int                 # H
    dk: int
    dv: int
    chunk: int                 # chunk size C of the prefill
    dtype: torch.dtype         # dtype of q, k, v and o
    alpha_mu: float            # mean of the pre-sigmoid decay logits
    s0_std: float              # 0 -> S0 = 0
    packed_seqs: int = 0       # >0: number of packed sequences (B == 1)
    max_len: int = 0           # packed: lengths uniform in [1, max_len]
    decode_steps: int = 0      # >0: a decode workload of this many steps
    decode_seqs: int = 0       # N sequences of the decode workload


# The workloads by name (the value is also the seed offset of each).
TINY_FP32, BATCHED_PREFILL, LONG_CONTEXT_PREFILL, DECODE, PACKED_VARLEN_RESUME = 0, 1, 2, 3, 4

CONFIGS = {
    0: Workload("tiny-fp32", 0, batch=1, seqlen=64, heads=1, dk=16, dv=16, chunk=16,
                dtype=torch.float32, alpha_mu=3.0, s0_std=0.0),
    1: Workload("batched-prefill", 1, batch=2, seqlen=2048, heads=4, dk=128, dv=128, chunk=64,
                dtype=torch.bfloat16, alpha_mu=3.0, s0_std=0.0),
    2: Workload("long-context-prefill", 2, batch=1, seqlen=65536, heads=32, dk=128, dv=128,
                chunk=64, dtype=torch.bfloat16, alpha_mu=4.0, s0_std=0.0),
    3: Workload("decode", 3, batch=1, seqlen=1, heads=32, dk=128, dv=128, chunk=64,
                dtype=torch.bfloat16, alpha_mu=3.0, s0_std=0.02,
                decode_steps=128, decode_seqs=256),
    4: Workload("packed-varlen-resume", 4, batch=1, seqlen=0, heads=16, dk=128, dv=128,
                chunk=64, dtype=torch.bfloat16, alpha_mu=3.0, s0_std=0.02,
                packed_seqs=64, max_len=32768),
}


def _rows_view(x: torch.Tensor, rows: int) -> torch.Tensor:
    return x.view(rows, x.numel() // rows if rows else 0)


def _randn(gen: torch.Generator, shape, rows: int) -> torch.Tensor:
    """N(0,1) fp32 of ``shape`` whose first axis has ``rows`` entries, drawn block by block."""
    out = torch.empty(shape, dtype=torch.float32)
    flat = _rows_view(out, rows)
    for r0 in range(0, rows, _BLOCK_TOKENS):
        r1 = min(rows, r0 + _BLOCK_TOKENS)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=gen, dtype=torch.float32)
    return out


def _l2norm_(x: torch.Tensor, rows: int) -> None:
    if rows == 0:
        return
    flat = x.view(rows, -1, x.shape[-1])
    for r0 in range(0, rows, _BLOCK_TOKENS):
        blk = flat[r0:r0 + _BLOCK_TOKENS]
        blk.div_(blk.norm(dim=-1, keepdim=True).clamp_min(1e-12))


def _cast(x: torch.Tensor, dtype: torch.dtype, rows: int) -> torch.Tensor:
    if dtype == torch.float32:
        return x
    out = torch.empty(x.shape, dtype=dtype)
    fo, fx = _rows_view(out, rows), _rows_view(x, rows)
    for r0 in range(0, rows, _BLOCK_TOKENS):
        fo[r0:r0 + _BLOCK_TOKENS] = fx[r0:r0 + _BLOCK_TOKENS].to(dtype)
    return out


def packed_lengths(gen: torch.Generator, n: int, max_len: int) -> torch.Tensor:
    """Sequence lengths uniform in [1, max_len] (int64)."""
    return torch.randint(1, max_len + 1, (n,), generator=gen, dtype=torch.int64)


def make_inputs(batch: int, seqlen: int, heads: int, dk: int, dv: int, dtype: torch.dtype,
                alpha_mu: float = 3.0, s0_std: float = 0.0, seed: int = 0,
                lengths: Optional[list] = None, num_state_seqs: Optional[int] = None):
    """Draw one set of KDA inputs on the CPU.

    Returns a dict with q, k, v ([B, T, H, d*], ``dtype``), alpha ([B, T, H, dk]
    fp32), beta ([B, T, H] fp32), S0 ([N, H, dk, dv] fp32 or None) and
    cu_seqlens (int32 [N+1] or None).  With ``lengths`` given the sequences are
    packed along T of a single row (B must be 1) and cu_seqlens describes them.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    cu = None
    if lengths is not None:
        assert batch == 1
        lens = torch.as_tensor(lengths, dtype=torch.int64)
        cu = torch.zeros(len(lens) + 1, dtype=torch.int64)
        cu[1:] = torch.cumsum(lens, 0)
        seqlen = int(cu[-1])
        n_seq = len(lens)
    else:
        n_seq = batch
    if num_state_seqs is not None:
        n_seq = num_state_seqs
    rows = batch * seqlen
    q = _randn(gen, (batch, seqlen, heads, dk), rows)
    _l2norm_(q, rows)
    q = _cast(q, dtype, rows)
    k = _randn(gen, (batch, seqlen, heads, dk), rows)
    _l2norm_(k, rows)
    k = _cast(k, dtype, rows)
    v = _randn(gen, (batch, seqlen, heads, dv), rows)
    fv = _rows_view(v, rows)
    for r0 in range(0, rows, _BLOCK_TOKENS):
        fv[r0:r0 + _BLOCK_TOKENS] = torch.nn.functional.silu(fv[r0:r0 + _BLOCK_TOKENS])
    v = _cast(v, dtype, rows)
    alpha = _randn(gen, (batch, seqlen, heads, dk), rows)
    fa = _rows_view(alpha, rows)
    for r0 in range(0, rows, _BLOCK_TOKENS):
        fa[r0:r0 + _BLOCK_TOKENS] = torch.sigmoid(fa[r0:r0 + _BLOCK_TOKENS] + alpha_mu)
    beta = torch.sigmoid(_randn(gen, (batch, seqlen, heads), rows))
    s0 = None
    if s0_std > 0.0:
        s0 = _randn(gen, (n_seq, heads, dk, dv), n_seq) * s0_std
    return {
        "q": q, "k": k, "v": v, "alpha": alpha, "beta": beta, "S0": s0,
        "cu_seqlens": None if cu is None else cu.to(torch.int32),
    }


def config_inputs(index: int, lengths_only: bool = False):
    """Inputs of prefill workload ``index`` (0, 1, 2 or 4)."""
    w = CONFIGS[index]
    assert w.decode_steps == 0
    seed = SEED_BASE + index
    lengths = None
    if w.packed_seqs:
        gen = torch.Generator(device="cpu")
        gen.manual_seed(seed)
        lengths = packed_lengths(gen, w.packed_seqs, w.max_len).tolist()
        if lengths_only:
            return lengths
        seed = seed + 1000  # the tensor draws follow from a second stream
    return make_inputs(w.batch, w.seqlen, w.heads, w.dk, w.dv, w.dtype, w.alpha_mu, w.s0_std,
                       seed=seed, lengths=lengths)


def decode_inputs(index: int = 3, steps: Optional[int] = None, seqs: Optional[int] = None):
    """Decode workload: S0 [N, H, dk, dv] and per-step q, k, v [steps, N, H, d], alpha, beta.

    The steps are drawn as one [N, steps] block of tokens, step-major on the
    way out so that step ``t`` is the contiguous slice ``[t]``.
    """
    w = CONFIGS[index]
    steps = w.decode_steps if steps is None else steps
    n = w.decode_seqs if seqs is None else seqs
    d = make_inputs(steps, n, w.heads, w.dk, w.dv, w.dtype, w.alpha_mu, 0.0,
                    seed=SEED_BASE + index)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(SEED_BASE + index + 500)
    s0 = _randn(gen, (n, w.heads, w.dk, w.dv), n) * w.s0_std
    # make_inputs draws [batch=steps, seqlen=n, ...]: axis 0 is the step.
    return {"q": d["q"], "k": d["k"], "v": d["v"], "alpha": d["alpha"], "beta": d["beta"],
            "S0": s0}


def device_inputs(index: int, device, seed_offset: int = 7000):
    """Inputs shaped like prefill workload ``index``, drawn directly on ``device``.

    Same shapes, dtypes and distributions as ``config_inputs(index)`` (and, for
    the packed workload, the very same sequence lengths, drawn on the CPU from
    the workload's seed), but the tensor values come from a device generator,
    so they differ from the CPU draw.  For timing runs, where drawing a
    million-token workload on the host would dominate the run.
    """
    w = CONFIGS[index]
    assert w.decode_steps == 0
    cu = None
    if w.packed_seqs:
        gen = torch.Generator(device="cpu")
        gen.manual_seed(SEED_BASE + index)
        lens = packed_lengths(gen, w.packed_seqs, w.max_len)
        cu = torch.zeros(len(lens) + 1, dtype=torch.int64)
        cu[1:] = torch.cumsum(lens, 0)
        batch, seqlen, n_seq = 1, int(cu[-1]), len(lens)
    else:
        batch, seqlen, n_seq = w.batch, w.seqlen, w.batch
    g = torch.Generator(device=device)
    g.manual_seed(SEED_BASE + index + seed_offset)
    shp = (batch, seqlen, w.heads)

    def unit(d):
        x = torch.randn(*shp, d, generator=g, device=device)
        return (x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)).to(w.dtype)

    q, k = unit(w.dk), unit(w.dk)
    v = torch.nn.functional.silu(torch.randn(*shp, w.dv, generator=g, device=device)).to(w.dtype)
    alpha = torch.sigmoid(torch.randn(*shp, w.dk, generator=g, device=device) + w.alpha_mu)
    beta = torch.sigmoid(torch.randn(*shp, generator=g, device=device))
    s0 = None
    if w.s0_std > 0.0:
        s0 = torch.randn(n_seq, w.heads, w.dk, w.dv, generator=g, device=device) * w.s0_std
    return {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta, "S0": s0,
            "cu_seqlens": None if cu is None else cu.to(torch.int32).to(device)}



def device_shape_inputs(seqlen: int, heads: int, dk: int, dv: int, dtype: torch.dtype, device,
                        alpha_mu: float = 4.0, s0_std: float = 0.0, seed: int = 0, slab: int = 65536):
    """One sequence (B = 1) of the recipe above drawn directly on ``device``, slab
    by slab of ``slab`` tokens so that the fp32 draws stay small next to the
    result (a million-token sequence over 32 heads holds 2^32 values per q).
    Values come from a device generator seeded with ``seed``."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = torch.empty(1, seqlen, heads, dk, dtype=dtype, device=device)
    k = torch.empty_like(q)
    v = torch.empty(1, seqlen, heads, dv, dtype=dtype, device=device)
    alpha = torch.empty(1, seqlen, heads, dk, dtype=torch.float32, device=device)
    beta = torch.empty(1, seqlen, heads, dtype=torch.float32, device=device)
    for t0 in range(0, seqlen, slab):
        n = min(slab, seqlen - t0)
        for dst in (q, k):
            x = torch.randn(1, n, heads, dk, generator=g, device=device)
            dst[:, t0:t0 + n] = (x / x.norm(dim=-1, keepdim=True).clamp_min(1e-12)).to(dtype)
        v[:, t0:t0 + n] = torch.nn.functional.silu(torch.randn(1, n, heads, dv, generator=g, device=device)).to(dtype)
        alpha[:, t0:t0 + n] = torch.sigmoid(torch.randn(1, n, heads, dk, generator=g, device=device) + alpha_mu)
        beta[:, t0:t0 + n] = torch.sigmoid(torch.randn(1, n, heads, generator=g, device=device))
    s0 = None
    if s0_std > 0.0:
        s0 = torch.randn(1, heads, dk, dv, generator=g, device=device) * s0_std
    return {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta, "S0": s0, "cu_seqlens": None}
