"""Parity of the HIP path (through the C ABI of libkda.so) against the fp64 oracle.

Error measure: max |gpu - oracle| / rms(oracle) over a whole tensor, for the
outputs o and the final states separately.  Bounds: 1e-4 for fp32 inputs and
2e-2 for bf16 inputs.  The bound is taken on o emitted in fp32: rounding a
perfectly computed o to bf16 alone already costs about 2.5e-2 in this
measure (tests/test_output_rounding.py), so the bf16 output is checked
separately: it must equal the fp32 output of the same launch configuration
rounded to nearest even, bit for bit.
"""
import numpy as np
import pytest
import torch

import linear_attention_sequence_gated_amd as kda
import workloads
from oracle import kda_oracle
from parity_measure import WholeTensorError, rel_err

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def say(*a):
    print(*a, flush=True)


def to_dev(inp):
    return {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_prefill(inp, chunk, scale=1.0, o_dtype=torch.float32, raw=False, **kw):
    d = to_dev(inp)
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"],
                         chunk_size=chunk, scale=scale, o_dtype=o_dtype, **kw)
    torch.cuda.synchronize()
    if raw:
        return o.cpu(), S.cpu()
    return o.float().cpu().numpy(), S.cpu().numpy()


def check_bf16_output(inp, chunk, scale=1.0):
    """bf16 o == RNE(fp32 o) of the same computation, bit for bit."""
    o32, _ = gpu_prefill(inp, chunk, scale, o_dtype=torch.float32, raw=True)
    o16, _ = gpu_prefill(inp, chunk, scale, o_dtype=torch.bfloat16, raw=True)
    assert o16.dtype == torch.bfloat16
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))


def oracle_prefill(inp, scale=1.0, heads=None):
    cu = inp["cu_seqlens"]
    return kda_oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                              cu_seqlens=None if cu is None else cu.to(torch.int64), scale=scale,
                              heads=heads)


def check(inp, chunk, tol, scale=1.0, label=""):
    say(f"[case] {label} chunk={chunk} q={tuple(inp['q'].shape)} {inp['q'].dtype}")
    og, Sg = gpu_prefill(inp, chunk, scale)
    oo, So = oracle_prefill(inp, scale)
    eo, es = rel_err(og, oo), rel_err(Sg, So)
    say(f"    err o={eo:.3e} S={es:.3e} (tol {tol})")
    assert eo < tol and es < tol, (eo, es)
    return eo, es


# --- the five workloads ------------------------------------------------------

def test_tiny_fp32_workload():
    w = workloads.CONFIGS[workloads.TINY_FP32]
    check(workloads.config_inputs(workloads.TINY_FP32), w.chunk, TOL[w.dtype], label=w.name)


def test_batched_prefill_bf16():
    w = workloads.CONFIGS[workloads.BATCHED_PREFILL]
    inp = workloads.config_inputs(workloads.BATCHED_PREFILL)
    check(inp, w.chunk, TOL[w.dtype], label=w.name)
    check_bf16_output(inp, w.chunk)


def whole_prefill_parity(inp, chunk, heads_per_group, label):
    """Every head of a full-size launch against the oracle, one group of heads at a time."""
    H = inp["q"].shape[2]
    say(f"[case] {label} GPU prefill, T={inp['q'].shape[1]} H={H}")
    d = to_dev(inp)
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"],
                         chunk_size=chunk, o_dtype=torch.float32)
    torch.cuda.synchronize()
    del d
    eo, es = WholeTensorError(), WholeTensorError()
    for h0 in range(0, H, heads_per_group):
        h1 = min(H, h0 + heads_per_group)
        say(f"[case] {label} oracle heads {h0}..{h1 - 1}")
        oo, So = oracle_prefill(inp, heads=(h0, h1))
        eo.add(o[:, :, h0:h1].contiguous().cpu().numpy(), oo)
        es.add(S[:, h0:h1].contiguous().cpu().numpy(), So)
        del oo, So
    say(f"    all {H} heads: err o={eo.value():.3e} S={es.value():.3e}")
    return eo.value(), es.value()


@pytest.mark.timeout(900)
def test_long_context_prefill_every_head():
    """Full-size launch (B1 H32 T65536): o and the final states of all 32 heads against the oracle."""
    w = workloads.CONFIGS[workloads.LONG_CONTEXT_PREFILL]
    say("[case] long-context-prefill generating inputs")
    inp = workloads.config_inputs(workloads.LONG_CONTEXT_PREFILL)
    eo, es = whole_prefill_parity(inp, w.chunk, 16, "long-context-prefill")
    assert eo < TOL[w.dtype] and es < TOL[w.dtype], (eo, es)


@pytest.mark.timeout(1200)
def test_packed_varlen_resume_every_head():
    """64 packed sequences (lengths U[1, 32768]), S0 != 0: all 16 heads against the oracle."""
    w = workloads.CONFIGS[workloads.PACKED_VARLEN_RESUME]
    say("[case] packed-varlen-resume generating inputs")
    inp = workloads.config_inputs(workloads.PACKED_VARLEN_RESUME)
    eo, es = whole_prefill_parity(inp, w.chunk, 4, "packed-varlen-resume")
    assert eo < TOL[w.dtype] and es < TOL[w.dtype], (eo, es)


@pytest.mark.timeout(900)
def test_one_million_token_sequence_sampled_heads():
    """One sequence of 2^20 tokens over 32 heads (the pages' million-token
    context; q holds 2^32 values, so flattened indices pass 32 bits), drawn on
    the device with the long-context recipe and S0 ~ N(0, 0.02): the call takes
    8 chunk ranges of 2,048 chunks per head.  Heads 0 and 31 (the lowest and
    highest offsets) against the oracle over every token, o and final state."""
    T, H, d = 1 << 20, 32, 128
    say("[case] one sequence of 2^20 tokens, H32: drawing inputs on the device")
    dd = workloads.device_shape_inputs(T, H, d, d, torch.bfloat16, "cuda", alpha_mu=4.0, s0_std=0.02, seed=1170)
    plan = kda.chunk_plan(dd["q"], dd["v"])
    assert plan["range_chunks"] == 2048, plan
    o, S = kda.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], dd["S0"], None, o_dtype=torch.float32)
    torch.cuda.synchronize()
    sample = [0, H - 1]
    inp = {n: dd[n][:, :, sample].contiguous().cpu() for n in ("q", "k", "v", "alpha", "beta")}
    inp["S0"] = dd["S0"][:, sample].contiguous().cpu()
    inp["cu_seqlens"] = None
    og = o[:, :, sample].contiguous().cpu().numpy()
    Sg = S[:, sample].contiguous().cpu().numpy()
    del dd, o, S
    torch.cuda.empty_cache()
    say("[case] one sequence of 2^20 tokens: oracle on heads 0 and 31")
    oo, So = oracle_prefill(inp)
    eo, es = rel_err(og, oo), rel_err(Sg, So)
    say(f"    heads 0, 31 over 2^20 tokens: err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16], (eo, es)


def _decode_run(inp, steps, scale=1.0, o_dtype=torch.float32):
    d = to_dev(inp)
    state = d["S0"].clone()
    outs = []
    for t in range(steps):
        outs.append(kda.decode_step(d["q"][t], d["k"][t], d["v"][t], d["alpha"][t], d["beta"][t], state,
                                    scale=scale, o_dtype=o_dtype))
    torch.cuda.synchronize()
    return torch.stack(outs).float().cpu().numpy(), state.cpu().numpy()


@pytest.mark.timeout(600)
def test_decode_128_steps_every_sequence():
    """256 sequences x H32, 128 in-place steps: o of every step and every final state against the oracle."""
    w = workloads.CONFIGS[workloads.DECODE]
    say("[case] decode generating inputs")
    inp = workloads.decode_inputs(3)
    say("[case] decode GPU decode x128")
    og, Sg = _decode_run(inp, w.decode_steps)
    say("[case] decode oracle, all 256 sequences")
    oo, So = kda_oracle.decode(inp["S0"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    eo, es = WholeTensorError(), WholeTensorError()
    eo.add(og, oo)
    es.add(Sg, So)
    say(f"    all sequences: err o={eo.value():.3e} S={es.value():.3e}")
    assert eo.value() < TOL[w.dtype] and es.value() < TOL[w.dtype], (eo.value(), es.value())


@pytest.mark.timeout(600)
def test_decode_state_past_32_bit_indices():
    """8,192 sequences x H32: the state holds 2^32 fp32 values (16 GiB), so its
    flattened indices pass 32 bits.  Two steps drawn on the device; sequences 0,
    4,095 and 8,191 (every head) against the oracle."""
    N, H, d, steps = 8192, 32, 128, 2
    g = torch.Generator(device="cuda").manual_seed(1180)
    say("[case] decode 8192 x H32, state of 2^32 values: drawing on the device")
    state = torch.randn(N, H, d, d, generator=g, device="cuda").mul_(0.02)
    sample = [0, N // 2 - 1, N - 1]
    S0 = state[sample].cpu()

    def unit():
        x = torch.randn(steps, N, H, d, generator=g, device="cuda")
        return (x / x.norm(dim=-1, keepdim=True)).to(torch.bfloat16)

    q, k = unit(), unit()
    v = torch.nn.functional.silu(torch.randn(steps, N, H, d, generator=g, device="cuda")).to(torch.bfloat16)
    alpha = torch.sigmoid(torch.randn(steps, N, H, d, generator=g, device="cuda") + 3.0)
    beta = torch.sigmoid(torch.randn(steps, N, H, generator=g, device="cuda"))
    outs = [kda.decode_step(q[t], k[t], v[t], alpha[t], beta[t], state, o_dtype=torch.float32)[sample].cpu()
            for t in range(steps)]
    torch.cuda.synchronize()
    og, Sg = torch.stack(outs).numpy(), state[sample].cpu().numpy()
    pick = lambda x: x[:, sample].cpu()
    oo, So = kda_oracle.decode(S0, pick(q), pick(k), pick(v), pick(alpha), pick(beta))
    eo, es = rel_err(og, oo), rel_err(Sg, So)
    say(f"    sequences {sample}: err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16], (eo, es)


# --- shapes, ragged tails, packing --------------------------------------------

SHAPES = [
    # B, T, H, dk, dv, C, dtype, S0
    (2, 100, 3, 64, 32, 32, torch.bfloat16, True),
    (1, 77, 2, 128, 128, 64, torch.float32, True),
    (3, 33, 1, 16, 128, 16, torch.bfloat16, False),
    (1, 200, 2, 32, 64, 64, torch.float32, False),
    (1, 1, 1, 128, 16, 64, torch.bfloat16, True),
    (2, 130, 2, 128, 64, 16, torch.float32, True),
    (1, 257, 2, 128, 128, 32, torch.bfloat16, True),
    # fp16 matrix-core tiles whose dk or C is 16 end in a single K=16 step next
    # to K=32 steps; dv >= 32 gives each compute wave two value slices
    (2, 70, 2, 32, 128, 16, torch.bfloat16, True),
    (1, 80, 2, 64, 128, 16, torch.bfloat16, True),
    (1, 90, 2, 16, 64, 32, torch.bfloat16, True),
    (1, 150, 1, 16, 32, 64, torch.bfloat16, False),
    # bf16, chunk 64, four channel groups in one wave: the paired 16-byte
    # workspace stores of the intra-chunk kernel with the fewest groups
    (1, 100, 2, 32, 64, 64, torch.bfloat16, True),
]


@pytest.mark.parametrize("B,T,H,dk,dv,C,dtype,s0", SHAPES)
def test_shapes(B, T, H, dk, dv, C, dtype, s0):
    inp = workloads.make_inputs(B, T, H, dk, dv, dtype, alpha_mu=3.0, s0_std=0.02 if s0 else 0.0,
                                seed=1000 + T + dk)
    check(inp, C, TOL[dtype], scale=0.75, label=f"shape B{B} T{T} H{H} dk{dk} dv{dv}")
    check_bf16_output(inp, C, scale=0.75)


def _random_case(seed):
    """A seeded random shape: batch or packed lengths (empty, one-token and
    partial-chunk sequences included), heads, dk, dv, chunk, dtype, initial
    state, decay level."""
    g = torch.Generator().manual_seed(seed)
    pick = lambda xs: xs[int(torch.randint(0, len(xs), (1,), generator=g))]
    dtype = pick([torch.bfloat16, torch.bfloat16, torch.float32])
    dk, dv, C = pick([16, 32, 64, 128]), pick([16, 32, 64, 128]), pick([16, 32, 64])
    H = int(torch.randint(1, 5, (1,), generator=g))
    s0 = pick([0.0, 0.02])
    if int(torch.randint(0, 2, (1,), generator=g)):
        lens = torch.randint(0, 300, (int(torch.randint(1, 9, (1,), generator=g)),), generator=g)
        lens[torch.rand(lens.shape, generator=g) < 0.2] = int(torch.randint(0, 2, (1,), generator=g))
        return dict(B=1, T=0, H=H, dk=dk, dv=dv, C=C, dtype=dtype, s0=s0, lengths=lens.tolist())
    return dict(B=int(torch.randint(1, 4, (1,), generator=g)), T=int(torch.randint(1, 400, (1,), generator=g)),
                H=H, dk=dk, dv=dv, C=C, dtype=dtype, s0=s0, lengths=None)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(seed):
    c = _random_case(4000 + seed)
    inp = workloads.make_inputs(c["B"], c["T"], c["H"], c["dk"], c["dv"], c["dtype"], s0_std=c["s0"],
                                seed=4100 + seed, lengths=c["lengths"])
    check(inp, c["C"], TOL[c["dtype"]], label=f"random {c}")


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_with_chunk_ranges(seed):
    """Seeded random long sequences over few heads (bf16, dk = dv in {64, 128}):
    fixed-length or packed with a long sequence among short and empty ones;
    every case takes the chunk-range path."""
    g = torch.Generator().manual_seed(6000 + seed)
    ri = lambda lo, hi: int(torch.randint(lo, hi, (1,), generator=g))
    d, H, s0 = [64, 128][ri(0, 2)], ri(1, 9), [0.0, 0.02][ri(0, 2)]
    if ri(0, 2):
        lens = [ri(0, 12000) if ri(0, 3) else ri(0, 200) for _ in range(ri(1, 6))]
        lens[ri(0, len(lens))] = ri(3072, 16000)
        B, T = 1, 0
    else:
        lens, B, T = None, ri(1, 3), ri(3072, 16384)
    inp = workloads.make_inputs(B, T, H, d, d, torch.bfloat16, s0_std=s0, seed=6100 + seed, lengths=lens)
    assert _ranged(B, T, H, d, lens)
    check(inp, 64, TOL[torch.bfloat16], label=f"random ranges B{B} T{T} H{H} d{d} lengths={lens}")


@pytest.mark.parametrize("seed", range(4))
def test_random_shapes_with_whole_rows(seed):
    """Seeded random packs with at least as many (sequence, head) pairs as CUs:
    whole-row workgroups, longest sequences first."""
    g = torch.Generator().manual_seed(7000 + seed)
    ri = lambda lo, hi: int(torch.randint(lo, hi, (1,), generator=g))
    H = [8, 16, 32][ri(0, 3)]
    lens = [ri(0, 700) for _ in range(256 // H + ri(1, 12))]
    dtype = [torch.bfloat16, torch.float32][ri(0, 2)]
    d = [64, 128][ri(0, 2)]
    inp = workloads.make_inputs(1, 0, H, d, d, dtype, s0_std=0.02, seed=7100 + seed, lengths=lens)
    cu = inp["cu_seqlens"].to("cuda")
    x = torch.empty(1, sum(lens), H, d, dtype=dtype, device="cuda")
    assert kda.chunk_plan(x, x, cu)["whole_rows"] == 1
    check(inp, 64, TOL[dtype], label=f"random whole rows H{H} d{d} {dtype} n={len(lens)}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_packed_ragged_with_empty_sequences(dtype):
    lens = [0, 1, 63, 64, 65, 200, 0, 129, 7]
    inp = workloads.make_inputs(1, 0, 2, 128, 128, dtype, s0_std=0.02, seed=77, lengths=lens)
    check(inp, 64, TOL[dtype], label=f"packed {lens}")


@pytest.mark.parametrize("C", [16, 32, 64])
def test_chunk_size_invariance(C):
    inp = workloads.make_inputs(2, 190, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=5)
    check(inp, C, TOL[torch.bfloat16], label="chunk invariance")


# --- degenerate gates ---------------------------------------------------------

def _gated(dtype, alpha_fn, beta_fn, T=150, seed=9):
    inp = workloads.make_inputs(1, T, 2, 128, 64, dtype, s0_std=0.02, seed=seed)
    inp["alpha"] = alpha_fn(inp["alpha"]).float().contiguous()
    inp["beta"] = beta_fn(inp["beta"]).float().contiguous()
    return inp


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_zero_decay_forgets_everything(dtype):
    inp = _gated(dtype, torch.zeros_like, lambda b: b)   # every chunk takes the exact pairwise path
    check(inp, 64, TOL[dtype], label="alpha=0")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fast_decay_exact_path(dtype):
    g = torch.Generator().manual_seed(3)
    inp = _gated(dtype, lambda a: torch.rand(a.shape, generator=g) * 0.2 + 0.05, lambda b: b)
    check(inp, 64, TOL[dtype], label="alpha in [0.05, 0.25]")


def test_mixed_zero_and_tiny_decay():
    g = torch.Generator().manual_seed(4)

    def alpha_fn(a):
        a = a.clone()
        m = torch.rand(a.shape, generator=g)
        a[m < 0.01] = 0.0
        a[(m >= 0.01) & (m < 0.02)] = 1e-30
        return a
    check(_gated(torch.float32, alpha_fn, lambda b: b), 64, TOL[torch.float32], label="sparse zeros")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_zero_beta_is_pure_decay(dtype):
    check(_gated(dtype, lambda a: a, torch.zeros_like), 64, TOL[dtype], label="beta=0")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("scale", [1.6, -0.5])
def test_beta_outside_unit_interval(dtype, scale):
    """beta is taken as given (no clamp): over-relaxed (beta up to 1.6) and negative
    update strengths, on both the factored and the exact Gram paths."""
    g = torch.Generator().manual_seed(31)
    fast = _gated(dtype, lambda a: a, lambda b: b * scale)
    check(fast, 64, TOL[dtype], label=f"beta x{scale}")
    exact = _gated(dtype, lambda a: torch.rand(a.shape, generator=g) * 0.2 + 0.05, lambda b: b * scale, seed=10)
    check(exact, 64, TOL[dtype], label=f"beta x{scale}, fast decay")


def test_identity_gate_keeps_state():
    inp = _gated(torch.float32, torch.ones_like, torch.zeros_like)
    og, Sg = gpu_prefill(inp, 64)
    np.testing.assert_allclose(Sg, inp["S0"].numpy(), rtol=0, atol=1e-6)
    ref = np.einsum("bthc,bhcj->bthj", inp["q"].double().numpy(), inp["S0"].double().numpy())
    assert rel_err(og, ref) < 1e-4


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_exact_recall_standard_basis_keys(dtype):
    """q = k = e_{i_t}, beta = 1: o_t = v_t for any decay (exact in bf16 storage)."""
    T, H, d = 160, 2, 128
    g = torch.Generator().manual_seed(11)
    idx = torch.randint(0, d, (1, T, H), generator=g)
    k = torch.nn.functional.one_hot(idx, d).to(dtype)
    inp = workloads.make_inputs(1, T, H, d, d, dtype, s0_std=0.02, seed=12)
    inp.update(q=k.clone(), k=k, beta=torch.ones(1, T, H))
    og, _ = gpu_prefill(inp, 64)
    err = rel_err(og, inp["v"].double().numpy())
    say(f"    recall err {err:.3e}")
    assert err < TOL[dtype]


# --- state plumbing -------------------------------------------------------------

def test_resume_from_final_state_equals_one_pass():
    inp = workloads.make_inputs(1, 300, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=21)
    o_full, S_full = gpu_prefill(inp, 64)
    cut = 131  # mid-chunk
    first = {k: (v[:, :cut].contiguous() if k in ("q", "k", "v", "alpha", "beta") else v)
             for k, v in inp.items()}
    o1, S1 = gpu_prefill(first, 64)
    second = {k: (v[:, cut:].contiguous() if k in ("q", "k", "v", "alpha", "beta") else v)
              for k, v in inp.items()}
    second["S0"] = torch.from_numpy(S1)
    o2, S2 = gpu_prefill(second, 64)
    assert rel_err(np.concatenate([o1, o2], axis=1), o_full) < 2e-2
    assert rel_err(S2, S_full) < 2e-2


def test_in_place_state_alias():
    inp = workloads.make_inputs(1, 129, 2, 64, 64, torch.float32, s0_std=0.02, seed=22)
    d = to_dev(inp)
    state = d["S0"].clone()
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], state, None, chunk_size=32,
                         final_state=state)
    torch.cuda.synchronize()
    assert S.data_ptr() == state.data_ptr()
    oo, So = oracle_prefill(inp)
    assert rel_err(state.cpu().numpy(), So) < 1e-4
    assert rel_err(o.cpu().numpy(), oo) < 1e-4


def test_empty_sequence_axis_copies_state():
    inp = workloads.make_inputs(2, 0, 2, 32, 32, torch.float32, s0_std=0.02, seed=23)
    og, Sg = gpu_prefill(inp, 32)
    np.testing.assert_array_equal(Sg, inp["S0"].numpy())
    assert og.size == 0


# --- decode --------------------------------------------------------------------

@pytest.mark.parametrize("dk,dv,dtype", [(128, 128, torch.bfloat16), (64, 32, torch.float32),
                                         (16, 128, torch.float32), (128, 16, torch.bfloat16)])
def test_decode_small(dk, dv, dtype):
    steps, N, H = 9, 3, 2
    inp = workloads.make_inputs(steps, N, H, dk, dv, dtype, seed=31 + dk)
    g = torch.Generator().manual_seed(32)
    inp["S0"] = torch.randn(N, H, dk, dv, generator=g) * 0.02
    say(f"[case] decode dk{dk} dv{dv} {dtype}")
    og, Sg = _decode_run(inp, steps, scale=1.3)
    oo, So = kda_oracle.decode(inp["S0"], inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                               scale=1.3)
    eo, es = rel_err(og, oo), rel_err(Sg, So)
    say(f"    err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[dtype] and es < TOL[dtype]
    ob, _ = _decode_run(inp, steps, scale=1.3, o_dtype=torch.bfloat16)
    assert np.array_equal(ob, torch.from_numpy(og).to(torch.bfloat16).float().numpy())


def test_decode_steps_equal_prefill():
    """T decode steps and one prefill over the same T tokens agree (GPU against GPU)."""
    steps, N, H, d = 70, 2, 2, 128
    inp = workloads.make_inputs(steps, N, H, d, d, torch.float32, seed=41)
    g = torch.Generator().manual_seed(42)
    inp["S0"] = torch.randn(N, H, d, d, generator=g) * 0.02
    od, Sd = _decode_run(inp, steps)
    pre = {k: (v.transpose(0, 1).contiguous() if k in ("q", "k", "v", "alpha", "beta") else v)
           for k, v in inp.items()}
    op, Sp = gpu_prefill(pre, 64)
    assert rel_err(od, op.transpose(1, 0, 2, 3)) < 1e-4
    assert rel_err(Sd, Sp) < 1e-4


def test_split_phases_equal_fused_call():
    """kda_chunk_fwd_intra then kda_chunk_fwd_inter is exactly kda_chunk_fwd."""
    inp = workloads.make_inputs(1, 300, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=51,
                                lengths=None)
    d = to_dev(inp)
    pre = kda.Prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], None, chunk_size=64,
                      o_dtype=torch.float32)
    o1, S1 = pre.run()
    o1, S1 = o1.clone(), S1.clone()
    pre.o.zero_()
    pre.intra()
    o2, S2 = pre.inter()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


# --- state checkpoints (kda_chunk_fwd_ex) ---------------------------------------

def _ckpt_check(inp, chunk, every, mx, tol, label):
    say(f"[case] checkpoints {label} chunk={chunk} every={every} max={mx} {inp['q'].dtype}")
    d = to_dev(inp)
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    n = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    ck = torch.full((n, mx, H, dk, dv), float("nan"), device="cuda")
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"],
                         chunk_size=chunk, o_dtype=torch.float32, checkpoints=ck, ckpt_every=every)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"]
    oo, So, cko = kda_oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                                     cu_seqlens=None if cu is None else cu.to(torch.int64),
                                     ckpt_every=every, max_ckpts=mx, return_ckpt=True)
    ckg = ck.cpu().numpy()
    written_g = ~np.isnan(ckg).all(axis=(2, 3, 4))
    written_o = ~np.isnan(cko).all(axis=(2, 3, 4))
    assert np.array_equal(written_g, written_o), (written_g, written_o)   # the same slots, the rest untouched
    assert written_o.any()
    worst = 0.0
    for sq, j in zip(*np.nonzero(written_o)):
        worst = max(worst, rel_err(ckg[sq, j], cko[sq, j]))
    eo, es = rel_err(o.cpu().numpy(), oo), rel_err(S.cpu().numpy(), So)
    say(f"    {int(written_o.sum())} checkpoints, err ckpt={worst:.3e} o={eo:.3e} S={es:.3e} (tol {tol})")
    assert worst < tol and eo < tol and es < tol
    return ck


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_checkpoints_packed_ragged(dtype):
    lens = [0, 1, 63, 64, 65, 200, 128, 129, 7]
    inp = workloads.make_inputs(1, 0, 2, 128, 128, dtype, s0_std=0.02, seed=91, lengths=lens)
    _ckpt_check(inp, 64, 64, 3, TOL[dtype], f"packed {lens}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_checkpoints_fixed_length(chunk):
    inp = workloads.make_inputs(2, 300, 3, 64, 32, torch.bfloat16, s0_std=0.02, seed=92)
    _ckpt_check(inp, chunk, 128, 3, TOL[torch.bfloat16], "B2 T300")


def test_resume_from_checkpoint():
    inp = workloads.make_inputs(1, 320, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=93)
    ck = _ckpt_check(inp, 64, 128, 2, TOL[torch.bfloat16], "resume source")
    # prefill resumed from checkpoint 1 (token 256) on the remaining tokens
    tail = {k: (v[:, 256:].contiguous() if k in ("q", "k", "v", "alpha", "beta") else v) for k, v in inp.items()}
    d = to_dev(tail)
    o2, S2 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ck[:, 1].contiguous(), None,
                           chunk_size=64, o_dtype=torch.float32)
    torch.cuda.synchronize()
    oo, So = oracle_prefill(inp)
    eo, es = rel_err(o2.cpu().numpy(), oo[:, 256:]), rel_err(S2.cpu().numpy(), So)
    say(f"    resumed tail err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16]


# --- decode options (kda_decode_step_ex) ----------------------------------------

def _decode_opts_case(N, H, dk, dv, steps, dtype, seed, pool=None, slots=None, **opts):
    """Run `steps` decode steps with options on the GPU and the oracle; return the errors."""
    g = torch.Generator().manual_seed(seed)
    fuse = opts.get("fuse_inputs", False)
    scal = opts.get("alpha_scalar", False)
    q = torch.randn(steps, N, H, dk, generator=g)
    k = torch.randn(steps, N, H, dk, generator=g)
    if not fuse:
        q = torch.nn.functional.normalize(q, dim=-1)
        k = torch.nn.functional.normalize(k, dim=-1)
    v = torch.nn.functional.silu(torch.randn(steps, N, H, dv, generator=g))
    a_shape = (steps, N, H) if scal else (steps, N, H, dk)
    al = torch.randn(*a_shape, generator=g) + 3.0          # logits
    bl = torch.randn(steps, N, H, generator=g)
    alpha, beta = (al, bl) if fuse else (torch.sigmoid(al), torch.sigmoid(bl))
    gate = torch.randn(steps, N, H, dv, generator=g).to(dtype) if opts.get("gate") else None
    w = (torch.rand(dv, generator=g) + 0.5) if opts.get("gate") else None
    q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    P = pool if pool is not None else N
    S0 = 0.02 * torch.randn(P, H, dk, dv, generator=g)
    floor = opts.get("decay_floor", 0.0)
    eps = 1e-5 if gate is not None else 0.0
    state = S0.cuda()
    dsl = None if slots is None else torch.tensor(slots, dtype=torch.int32, device="cuda")
    outs = []
    for t in range(steps):
        o = kda.decode_step(q[t].cuda(), k[t].cuda(), v[t].cuda(), alpha[t].cuda(), beta[t].cuda(), state,
                            o_dtype=torch.float32, state_slots=dsl, decay_floor=floor, alpha_scalar=scal,
                            fuse_inputs=fuse, gate=None if gate is None else gate[t].cuda(),
                            norm_weight=None if w is None else w.cuda(), norm_eps=eps)
        outs.append(o)
    torch.cuda.synchronize()
    og = torch.stack(outs).cpu().numpy()
    oo, So = kda_oracle.decode(S0, q, k, v, alpha, beta, state_slots=slots, decay_floor=floor,
                               alpha_scalar=scal, fuse_inputs=fuse, gate=gate, norm_weight=w, norm_eps=eps)
    sg = state.cpu()
    idx = list(range(N)) if slots is None else list(slots)
    eo, es = rel_err(og, oo), rel_err(sg[idx].numpy(), So)
    if slots is not None:   # pool entries outside the call are untouched, bit for bit
        rest = [p for p in range(P) if p not in slots]
        assert torch.equal(sg[rest], S0[rest])
    return eo, es


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_paged_state_pool(dtype):
    say(f"[case] decode paged pool {dtype}")
    eo, es = _decode_opts_case(4, 3, 128, 128, 5, dtype, seed=301, pool=7, slots=[5, 0, 3, 6])
    say(f"    err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[dtype] and es < TOL[dtype]


@pytest.mark.parametrize("gated", [False, True])
def test_decode_slot_outside_the_pool_is_skipped(gated):
    """A slot outside [0, P) is caught on the device: that sequence's o reads NaN and no
    state is touched; the other sequences step as usual.  The pool tensor has one
    padding entry beyond the P entries declared, so even an unchecked step would stay
    inside the allocation (slot P is that padding entry)."""
    N, H, d, P = 3, 2, 128, 4
    g = torch.Generator().manual_seed(330)
    q = torch.nn.functional.normalize(torch.randn(N, H, d, generator=g), dim=-1).to(torch.bfloat16)
    k = torch.nn.functional.normalize(torch.randn(N, H, d, generator=g), dim=-1).to(torch.bfloat16)
    v = torch.nn.functional.silu(torch.randn(N, H, d, generator=g)).to(torch.bfloat16)
    alpha = torch.sigmoid(torch.randn(N, H, d, generator=g) + 3.0)
    beta = torch.sigmoid(torch.randn(N, H, generator=g))
    gate = torch.randn(N, H, d, generator=g).to(torch.bfloat16) if gated else None
    pool0 = 0.02 * torch.randn(P + 1, H, d, d, generator=g)
    slots = [2, P, 0]                          # sequence 1 points past the declared pool
    say(f"[case] decode slot outside the pool, gated={gated}")
    pool = pool0.cuda()
    o = kda.decode_step(q.cuda(), k.cuda(), v.cuda(), alpha.cuda(), beta.cuda(), pool, o_dtype=torch.float32,
                        state_slots=torch.tensor(slots, dtype=torch.int32, device="cuda"), pool_entries=P,
                        gate=None if gate is None else gate.cuda(), norm_eps=1e-5 if gated else 0.0)
    torch.cuda.synchronize()
    o, pool = o.cpu(), pool.cpu()
    assert torch.isnan(o[1]).all() and torch.isfinite(o[[0, 2]]).all()
    assert torch.equal(pool[[1, 3, P]], pool0[[1, 3, P]])       # unused and padding entries untouched
    good = [0, 2]
    oo, So = kda_oracle.decode(pool0[[slots[n] for n in good]], q[None, good], k[None, good], v[None, good],
                               alpha[None, good], beta[None, good], gate=None if gate is None else gate[None, good],
                               norm_eps=1e-5 if gated else 0.0)
    assert rel_err(o[good].numpy(), oo[0]) < TOL[torch.bfloat16]
    assert rel_err(pool[[slots[n] for n in good]].numpy(), So) < TOL[torch.bfloat16]


DECODE_OPTS = [
    {"decay_floor": 0.97},
    {"alpha_scalar": True},
    {"fuse_inputs": True},
    {"gate": True},
    {"fuse_inputs": True, "gate": True, "decay_floor": 0.9},
    {"fuse_inputs": True, "alpha_scalar": True, "gate": True},
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("opts", DECODE_OPTS, ids=lambda o: "+".join(sorted(o)))
def test_decode_options(opts, dtype):
    for (dk, dv) in ((128, 128), (64, 32)):
        say(f"[case] decode options {opts} {dtype} dk={dk} dv={dv}")
        eo, es = _decode_opts_case(6, 4, dk, dv, 4, dtype, seed=310 + dk + dv, **opts)
        say(f"    err o={eo:.3e} S={es:.3e}")
        assert eo < TOL[dtype] and es < TOL[dtype]


def test_decode_options_combined_with_pool():
    say("[case] decode pool + fused inputs + gate + floor")
    eo, es = _decode_opts_case(5, 2, 128, 64, 3, torch.bfloat16, seed=333, pool=9, slots=[8, 1, 4, 0, 2],
                               fuse_inputs=True, gate=True, decay_floor=0.95)
    say(f"    err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16]


# --- prefill input options (kda_chunk_fwd_ex) -----------------------------------

def _prefill_opts_inputs(B, T, H, dk, dv, dtype, seed, lengths=None, alpha_mu=3.0, **opts):
    g = torch.Generator().manual_seed(seed)
    fuse = opts.get("fuse_inputs", False)
    scal = opts.get("alpha_scalar", False)
    tot = B * T if lengths is None else sum(lengths)
    sh = (B, T) if lengths is None else (1, tot)
    q = torch.randn(*sh, H, dk, generator=g) * 2.0
    k = torch.randn(*sh, H, dk, generator=g) * 0.7
    if not fuse:
        q = torch.nn.functional.normalize(q, dim=-1)
        k = torch.nn.functional.normalize(k, dim=-1)
    v = torch.nn.functional.silu(torch.randn(*sh, H, dv, generator=g))
    al = torch.randn(*sh, H, *(() if scal else (dk,)), generator=g) + alpha_mu
    bl = torch.randn(*sh, H, generator=g)
    n = B if lengths is None else len(lengths)
    inp = {"q": q.to(dtype), "k": k.to(dtype), "v": v.to(dtype),
           "alpha": al if fuse else torch.sigmoid(al), "beta": bl if fuse else torch.sigmoid(bl),
           "S0": 0.02 * torch.randn(n, H, dk, dv, generator=g),
           "cu_seqlens": None if lengths is None else
           torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)}
    return inp


def _prefill_opts_check(inp, chunk, tol, label, **opts):
    say(f"[case] prefill options {opts} {label} chunk={chunk} {inp['q'].dtype}")
    og, Sg = gpu_prefill(inp, chunk, **opts)
    cu = inp["cu_seqlens"]
    oo, So = kda_oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                                cu_seqlens=None if cu is None else cu.to(torch.int64), **opts)
    eo, es = rel_err(og, oo), rel_err(Sg, So)
    say(f"    err o={eo:.3e} S={es:.3e} (tol {tol})")
    assert eo < tol and es < tol


PREFILL_OPTS = [
    {"decay_floor": 0.9},
    {"alpha_scalar": True},
    {"fuse_inputs": True},
    {"fuse_inputs": True, "alpha_scalar": True, "decay_floor": 0.8},
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("opts", PREFILL_OPTS, ids=lambda o: "+".join(sorted(o)))
def test_prefill_options(opts, dtype):
    lens = [1, 63, 64, 65, 150, 7]
    inp = _prefill_opts_inputs(1, 0, 2, 128, 128, dtype, seed=401, lengths=lens, **opts)
    _prefill_opts_check(inp, 64, TOL[dtype], f"packed {lens}", **opts)
    inp = _prefill_opts_inputs(2, 100, 3, 64, 32, dtype, seed=402, **opts)
    _prefill_opts_check(inp, 16, TOL[dtype], "B2 T100 dk64 dv32", **opts)


@pytest.mark.parametrize("opts", [{"fuse_inputs": True}, {"alpha_scalar": True}, {"decay_floor": 0.01}],
                         ids=lambda o: "+".join(sorted(o)))
def test_prefill_options_fast_decay_exact_path(opts):
    # alpha ~ sigmoid(N(-3, 1)): 16-token blocks decay far beyond the factored
    # path's range, so chunks take the exact pairwise path
    inp = _prefill_opts_inputs(1, 200, 2, 128, 128, torch.bfloat16, seed=403, alpha_mu=-3.0, **opts)
    _prefill_opts_check(inp, 64, TOL[torch.bfloat16], "fast decay", **opts)


def test_prefill_options_with_checkpoints():
    lens = [200, 64, 130]
    opts = {"fuse_inputs": True, "decay_floor": 0.5}
    inp = _prefill_opts_inputs(1, 0, 2, 128, 64, torch.bfloat16, seed=404, lengths=lens, **opts)
    say(f"[case] prefill options + checkpoints {opts}")
    d = to_dev(inp)
    ck = torch.full((3, 3, 2, 128, 64), float("nan"), device="cuda")
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"], chunk_size=64,
                         o_dtype=torch.float32, checkpoints=ck, ckpt_every=64, **opts)
    torch.cuda.synchronize()
    oo, So, cko = kda_oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                                     cu_seqlens=inp["cu_seqlens"].to(torch.int64), ckpt_every=64, max_ckpts=3,
                                     return_ckpt=True, **opts)
    ckg = ck.cpu().numpy()
    wo = ~np.isnan(cko).all(axis=(2, 3, 4))
    assert np.array_equal(~np.isnan(ckg).all(axis=(2, 3, 4)), wo)
    worst = max(rel_err(ckg[a, b], cko[a, b]) for a, b in zip(*np.nonzero(wo)))
    eo, es = rel_err(o.cpu().numpy(), oo), rel_err(S.cpu().numpy(), So)
    say(f"    err ckpt={worst:.3e} o={eo:.3e} S={es:.3e}")
    assert worst < 2e-2 and eo < 2e-2 and es < 2e-2


# --- output norm and gate inside the inter-chunk kernel -------------------------

def _gate_case(inp, chunk, tol, label, o_dtype=torch.float32, misalign=False, **opts):
    say(f"[case] prefill gate {label} chunk={chunk} {inp['q'].dtype} {opts}")
    g = torch.Generator().manual_seed(int(inp["q"].shape[1]) + chunk)
    gate = torch.randn(inp["v"].shape, generator=g).to(inp["q"].dtype)
    w = torch.rand(inp["v"].shape[-1], generator=g) + 0.5
    eps = 1e-5
    d = to_dev(inp)
    gd, wd = gate.cuda(), w.cuda()
    if misalign:   # one element past an aligned allocation: only element alignment
        gbuf = torch.empty(gate.numel() + 1, dtype=gate.dtype, device="cuda")
        gbuf[1:].copy_(gd.reshape(-1))
        gd = gbuf[1:].view(gate.shape)
        wbuf = torch.empty(w.numel() + 1, device="cuda")
        wbuf[1:].copy_(wd)
        wd = wbuf[1:]
        assert gd.data_ptr() % (4 * gate.element_size()) != 0 and wd.data_ptr() % 16 != 0
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"],
                         chunk_size=chunk, o_dtype=o_dtype, gate=gd, norm_weight=wd, norm_eps=eps,
                         **opts)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"]
    oo, So = kda_oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                                cu_seqlens=None if cu is None else cu.to(torch.int64), gate=gate, norm_weight=w,
                                norm_eps=eps, **opts)
    eo, es = rel_err(o.float().cpu().numpy(), oo), rel_err(S.cpu().numpy(), So)
    say(f"    err o={eo:.3e} S={es:.3e} (tol {tol})")
    assert eo < tol and es < tol
    return o


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_gate_packed(dtype):
    lens = [1, 63, 64, 65, 150, 7]
    inp = workloads.make_inputs(1, 0, 2, 128, 128, dtype, s0_std=0.02, seed=501, lengths=lens)
    _gate_case(inp, 64, TOL[dtype], f"packed {lens}")


@pytest.mark.parametrize("dv,chunk", [(16, 32), (32, 16), (64, 64)])
def test_prefill_gate_shapes(dv, chunk):
    inp = workloads.make_inputs(2, 130, 3, 64, dv, torch.bfloat16, s0_std=0.02, seed=502 + dv)
    _gate_case(inp, chunk, TOL[torch.bfloat16], f"B2 T130 dk64 dv{dv}")


def test_prefill_gate_with_fused_inputs():
    opts = {"fuse_inputs": True, "decay_floor": 0.5}
    inp = _prefill_opts_inputs(1, 200, 2, 128, 128, torch.bfloat16, seed=503, **opts)
    _gate_case(inp, 64, TOL[torch.bfloat16], "B1 T200 fused", **opts)


def test_prefill_gate_bf16_output_is_rounded_fp32():
    inp = workloads.make_inputs(1, 100, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=504)
    o32 = _gate_case(inp, 64, TOL[torch.bfloat16], "fp32 out").cpu()
    o16 = _gate_case(inp, 64, 4e-2, "bf16 out", o_dtype=torch.bfloat16).cpu()
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_prefill_gate_unaligned_gate_and_weight(dtype):
    # few (sequence, head) pairs take the split path, whose epilogue reads the
    # gate logits and the norm weight as vectors only when the pointers allow:
    # offset views take its element-wise loads, with the same result
    inp = workloads.make_inputs(1, 150, 2, 128, 128, dtype, s0_std=0.02, seed=506)
    oa = _gate_case(inp, 64, TOL[dtype], "aligned").cpu()
    om = _gate_case(inp, 64, TOL[dtype], "gate and weight one element off", misalign=True).cpu()
    assert torch.equal(oa, om)


def test_prefill_gate_many_packed_sequences_whole_rows():
    # packed, at least as many pairs as CUs: whole rows in the longest-first
    # sequence order, norm and gate finished in the inter-chunk pass
    g = torch.Generator().manual_seed(507)
    lens = torch.randint(0, 200, (300,), generator=g).tolist()
    inp = workloads.make_inputs(1, 0, 1, 128, 128, torch.bfloat16, s0_std=0.02, seed=507, lengths=lens)
    _gate_case(inp, 64, TOL[torch.bfloat16], "300 packed sequences x H1")


def test_prefill_gate_many_units_fused_in_inter_kernel():
    # at least as many (sequence, head) pairs as CUs: the whole-row workgroups
    # apply the norm and gate inside the inter-chunk kernel
    inp = workloads.make_inputs(64, 70, 4, 64, 64, torch.bfloat16, s0_std=0.02, seed=505)
    _gate_case(inp, 32, TOL[torch.bfloat16], "B64 H4 (256 units)")


# --- whole-row inter-chunk workgroups ---------------------------------------------
# With at least as many (sequence, head) pairs as the device has CUs (256 on
# MI355X), every value slice of a row shares one inter-chunk workgroup.

@pytest.mark.parametrize("dk,dv,C,dtype", [(128, 128, 64, torch.bfloat16), (64, 32, 32, torch.bfloat16),
                                           (32, 64, 16, torch.float32), (128, 16, 64, torch.bfloat16),
                                           (128, 128, 32, torch.float32), (16, 128, 64, torch.bfloat16)])
def test_whole_row_workgroups(dk, dv, C, dtype):
    inp = workloads.make_inputs(64, 70, 4, dk, dv, dtype, s0_std=0.02, seed=600 + dk + dv + C)
    check(inp, C, TOL[dtype], label=f"256 units dk{dk} dv{dv}")
    check_bf16_output(inp, C)


def test_whole_row_packed_beyond_the_sequence_sort():
    # more packed sequences than the longest-first sort holds keep their input
    # order in the whole-row pass
    g = torch.Generator().manual_seed(611)
    lens = torch.randint(0, 40, (4100,), generator=g).tolist()
    inp = workloads.make_inputs(1, 0, 1, 64, 64, torch.bfloat16, s0_std=0.02, seed=611, lengths=lens)
    check(inp, 64, TOL[torch.bfloat16], label="4100 packed sequences x H1")


def test_whole_row_workgroups_packed_with_checkpoints():
    g = torch.Generator().manual_seed(610)
    lens = torch.randint(0, 200, (130,), generator=g).tolist()
    lens[:4] = [0, 1, 64, 129]
    inp = workloads.make_inputs(1, 0, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=611, lengths=lens)
    check(inp, 64, TOL[torch.bfloat16], label="130 packed sequences x H2")
    _ckpt_check(inp, 64, 64, 2, TOL[torch.bfloat16], "130 packed sequences x H2")


# --- scalar-gate and floored-decay instances of the intra-chunk kernel --------------

@pytest.mark.timeout(900)
def test_scalar_gate_long_context_every_head():
    """One decay per (token, head) at the long-context shape (B1 H32 T65536): every head against the oracle."""
    w = workloads.CONFIGS[workloads.LONG_CONTEXT_PREFILL]
    say("[case] scalar gate, long-context shape: generating inputs")
    inp = workloads.config_inputs(workloads.LONG_CONTEXT_PREFILL)
    inp["alpha"] = inp["alpha"][..., 0].contiguous()   # one sigmoid(N(4, 1)) draw per (token, head)
    d = to_dev(inp)
    o, S = kda.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None, None, chunk_size=w.chunk,
                         o_dtype=torch.float32, alpha_scalar=True)
    torch.cuda.synchronize()
    del d
    eo, es = WholeTensorError(), WholeTensorError()
    for h0 in range(0, 32, 16):
        say(f"[case] scalar gate oracle heads {h0}..{h0 + 15}")
        oo, So = kda_oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], heads=(h0, h0 + 16),
                                    alpha_scalar=True)
        eo.add(o[:, :, h0:h0 + 16].contiguous().cpu().numpy(), oo)
        es.add(S[:, h0:h0 + 16].contiguous().cpu().numpy(), So)
        del oo, So
    say(f"    all 32 heads: err o={eo.value():.3e} S={es.value():.3e}")
    assert eo.value() < TOL[w.dtype] and es.value() < TOL[w.dtype]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("alpha_mu", [3.0, -3.0])
def test_scalar_gate_shapes(dtype, alpha_mu):
    # alpha_mu = -3: the decay over a chunk spans far more than any fp16 factor
    # could hold; the scalar path's mask is formed in fp32 and needs no fallback
    for (B, T, H, dk, dv, C) in ((2, 150, 3, 128, 64, 64), (1, 97, 2, 64, 128, 32), (2, 70, 2, 32, 32, 16)):
        inp = _prefill_opts_inputs(B, T, H, dk, dv, dtype, seed=700 + T, alpha_mu=alpha_mu, alpha_scalar=True)
        _prefill_opts_check(inp, C, TOL[dtype], f"B{B} T{T} dk{dk} dv{dv}", alpha_scalar=True)


@pytest.mark.parametrize("floor", [0.59460356, 0.6, 0.95])
def test_decay_floor_fast_instance(floor):
    # floors at or above 2^-0.75 run the instance without the range check and
    # the exact path; with alpha ~ sigmoid(N(-3, 1)) nearly every value is floored
    for alpha_mu in (4.0, -3.0):
        lens = [1, 63, 64, 65, 300, 7, 128]
        inp = _prefill_opts_inputs(1, 0, 3, 128, 128, torch.bfloat16, seed=720, lengths=lens, alpha_mu=alpha_mu,
                                   decay_floor=floor)
        _prefill_opts_check(inp, 64, TOL[torch.bfloat16], f"packed {lens} mu {alpha_mu}", decay_floor=floor)


# --- range contract of the bf16 path (fp16 matrix-core operands) --------------------

def _large(dtype, v_scale=1.0, s0_scale=1.0, seed=900):
    inp = workloads.make_inputs(1, 200, 2, 128, 128, dtype, s0_std=0.02, seed=seed)
    inp["v"] = (inp["v"].float() * v_scale).to(dtype)
    inp["S0"] = inp["S0"] * s0_scale
    return inp


@pytest.mark.parametrize("v_scale,s0_scale", [(1e5, 1.0), (1.0, 5e6)])
def test_range_guard_reports_overflow(v_scale, s0_scale):
    """|v| or the state past the fp16 range: KDA_ERR_RANGE, never a silent inf; fp32 inputs compute it."""
    say(f"[case] range guard v x{v_scale:g} S0 x{s0_scale:g}")
    inp = _large(torch.bfloat16, v_scale, s0_scale)
    with pytest.raises(kda.KdaError) as e:
        gpu_prefill(inp, 64)
    assert e.value.status == kda.KDA_ERR_RANGE
    # the same values in fp32 inputs run in fp32 and match the oracle
    inp32 = _large(torch.float32, v_scale, s0_scale)
    check(inp32, 64, TOL[torch.float32], label=f"fp32 v x{v_scale:g} S0 x{s0_scale:g}")


def test_range_guard_large_values_inside_range():
    """Values well above 1 but inside the fp16 range compute normally and pass the status check."""
    check(_large(torch.bfloat16, v_scale=300.0, s0_scale=3000.0), 64, TOL[torch.bfloat16], label="v x300 S0 x3000")


def test_range_status_reads_clear_after_an_empty_call():
    """A call that writes no token (T = 0) leaves the status word clear even after an overflowing call."""
    inp = _large(torch.bfloat16, 1e5)
    d = to_dev(inp)
    pre = kda.Prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], None, chunk_size=64)
    pre.run()
    assert pre.status() == kda.KDA_ERR_RANGE
    e = {k: (v[:, :0].contiguous() if k in ("q", "k", "v", "alpha", "beta") else v) for k, v in d.items()}
    pre0 = kda.Prefill(e["q"], e["k"], e["v"], e["alpha"], e["beta"], e["S0"], None, chunk_size=64,
                       workspace=pre.workspace)
    pre0.run()
    assert pre0.status() == 0


# --- layout check of cu_seqlens on the device ----------------------------------------
# Each malformed array below keeps every offset inside the tensors, so even a
# call that did not check it would read and write in bounds.

@pytest.mark.parametrize("lens,bad", [
    ([100, 40, 60], [0, 100, 60, 200]),            # decreasing
    ([100, 40, 60], [0, 100, 150, 150]),           # cu[N] != T
    ([100, 40, 60], [10, 100, 150, 200]),          # cu[0] != 0
    ([5000, 4000], [0, 5000, 4500]),                # decreasing, on a shape with chunk ranges
])
def test_malformed_cu_seqlens_is_reported_and_writes_no_token(lens, bad):
    inp = workloads.make_inputs(1, 0, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=1320, lengths=lens)
    d = to_dev(inp)
    say(f"[case] malformed cu_seqlens {bad} for lengths {lens}")
    o = torch.full(d["v"].shape, float("nan"), dtype=torch.float32, device="cuda")
    pre = kda.Prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                      torch.tensor(bad, dtype=torch.int32, device="cuda"), chunk_size=64, o=o,
                      o_dtype=torch.float32)
    pre.run()
    with pytest.raises(kda.KdaError) as e:
        pre.check_range()
    assert e.value.status == kda.KDA_ERR_INVALID_ARG
    assert torch.isnan(o).all()
    # the well-formed call on the same workspace reads clear and matches the oracle
    good = kda.Prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"], chunk_size=64,
                       o_dtype=torch.float32, workspace=pre.workspace)
    og, Sg = good.run()
    assert good.status() == 0
    oo, So = oracle_prefill(inp)
    assert rel_err(og.cpu().numpy(), oo) < TOL[torch.bfloat16] and rel_err(Sg.cpu().numpy(), So) < TOL[torch.bfloat16]


# --- chunk-range scan (few (sequence, head) pairs, long sequences) -----------------
# With fewer pairs than CUs and at least three 16-chunk ranges per sequence the
# inter-chunk pass forms each range's map, scans the ranges' start states and
# runs the ranges side by side.

def _ranged(B, T, H, d, lengths=None):
    cu = None if lengths is None else torch.tensor(np.cumsum([0] + lengths), dtype=torch.int32, device="cuda")
    Tq = T if lengths is None else sum(lengths)
    x = torch.empty(B, Tq, H, d, dtype=torch.bfloat16, device="cuda")
    return kda.chunk_plan(x, x, cu)["range_chunks"] > 0


@pytest.mark.parametrize("B,T,H,d,lengths,expect", [
    (2, 5000, 2, 128, None, True), (1, 4096, 4, 64, None, True), (1, 6200, 3, 128, None, True),
    (1, 0, 2, 128, [9000, 0, 7000, 1, 3072], True), (1, 65536, 32, 128, None, True),
    (1, 3072, 4, 128, None, True),       # 48 chunks: three 16-chunk ranges
    (1, 3008, 4, 128, None, False),      # 47 chunks: fewer than three
    (1, 8192, 256, 64, None, False),     # as many pairs as CUs
])
def test_chunk_range_scan_selection(B, T, H, d, lengths, expect):
    if H >= 256 and torch.cuda.get_device_properties(0).multi_processor_count > 256:
        pytest.skip("device has more than 256 CUs")
    assert _ranged(B, T, H, d, lengths) == expect


@pytest.mark.parametrize("B,T,H,d", [(2, 5000, 2, 128), (1, 4096, 4, 64), (1, 6200, 3, 128)])
def test_chunk_range_scan_fixed_length(B, T, H, d):
    inp = workloads.make_inputs(B, T, H, d, d, torch.bfloat16, s0_std=0.02, seed=1100 + T + d)
    check(inp, 64, TOL[torch.bfloat16], label=f"ranges B{B} T{T} H{H} d{d}")
    check_bf16_output(inp, 64)


def test_chunk_range_scan_packed_with_empty_and_tiny_sequences():
    lens = [9000, 0, 7000, 1, 3072]
    inp = workloads.make_inputs(1, 0, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=1110, lengths=lens)
    check(inp, 64, TOL[torch.bfloat16], label=f"ranges packed {lens}")


def test_chunk_range_scan_checkpoints_cross_ranges():
    # 1024-token checkpoints land inside and at the ends of the 16-chunk ranges
    inp = workloads.make_inputs(1, 0, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=1111, lengths=[9000, 4100])
    _ckpt_check(inp, 64, 1024, 9, TOL[torch.bfloat16], "ranges packed [9000, 4100]")


@pytest.mark.parametrize("B,T,H,lengths", [(2, 5000, 2, None), (1, 0, 2, [9000, 0, 7000, 1, 3072])])
def test_chunk_range_scan_gated(B, T, H, lengths):
    # the output norm and gate are finished in the ranged whole-row pass
    inp = workloads.make_inputs(B, T, H, 128, 128, torch.bfloat16, s0_std=0.02, seed=1120 + T, lengths=lengths)
    assert _ranged(B, T, H, 128, lengths)
    _gate_case(inp, 64, TOL[torch.bfloat16], f"ranges B{B} T{T} H{H} {lengths}")


@pytest.mark.parametrize("dtype", [torch.bfloat16])
def test_chunk_range_scan_gated_unaligned_gate(dtype):
    # gate logits one element past an aligned allocation take element loads
    # in the whole-row pass; the result is the same bit for bit
    inp = workloads.make_inputs(2, 5000, 2, 128, 128, dtype, s0_std=0.02, seed=1123)
    assert _ranged(2, 5000, 2, 128)
    oa = _gate_case(inp, 64, TOL[dtype], "ranges aligned").cpu()
    om = _gate_case(inp, 64, TOL[dtype], "ranges gate and weight one element off", misalign=True).cpu()
    assert torch.equal(oa, om)


def test_chunk_range_scan_gated_fused_inputs():
    opts = {"fuse_inputs": True}
    inp = _prefill_opts_inputs(1, 6200, 3, 128, 128, torch.bfloat16, seed=1122, **opts)
    assert _ranged(1, 6200, 3, 128)
    _gate_case(inp, 64, TOL[torch.bfloat16], "ranges B1 T6200 H3 fused", **opts)


@pytest.mark.parametrize("opts", [{"decay_floor": 0.6}, {"alpha_scalar": True}, {"decay_floor": 0.3}])
def test_chunk_range_scan_with_input_options(opts):
    # the floor and scalar-gate instances of the intra-chunk kernel feed the
    # range maps and the ranged walk like the plain one
    lens = [9000, 6100, 0, 64]
    inp = _prefill_opts_inputs(1, 0, 2, 128, 128, torch.bfloat16, seed=1124, lengths=lens, alpha_mu=2.0, **opts)
    assert _ranged(1, 0, 2, 128, lens)
    _prefill_opts_check(inp, 64, TOL[torch.bfloat16], f"ranges packed {lens}", **opts)


# Long memory.  With decays drawn per token as sigmoid(N(3..4, 1)) a state
# forgets where it started within about a thousand tokens: the A part of a
# range map, A = prod (diag(gamma) - Kbar^T W), falls far below fp32
# resolution and a ranged call equals sequential calls bit for bit, so those
# inputs cannot tell a wrong A from a right one.  Here alpha = sigmoid(N(8, 1))
# (1 - alpha ~ 3e-4) and beta is scaled by 0.1, so a range's start state still
# moves the outputs two ranges (2,048 tokens) later by more than 10 % of their
# RMS (asserted on the oracle first): the maps' A and the scan's A S carry it.

def _long_memory_inputs(B, T, H, d, seed, lengths=None, alpha_mu=8.0, beta_scale=0.1):
    inp = workloads.make_inputs(B, T, H, d, d, torch.bfloat16, alpha_mu=alpha_mu, s0_std=0.05, seed=seed,
                                lengths=lengths)
    inp["beta"] = inp["beta"] * beta_scale
    return inp


def _assert_long_memory(inp, row_tokens, span=1024):
    """Row 0's last `span` outputs change by > 10 % of their RMS when the state
    3 `span` tokens before the end is replaced by zeros (oracle only)."""
    names = ("q", "k", "v", "alpha", "beta")
    cut = row_tokens - 3 * span
    head = {n: inp[n][:1, :cut] for n in names}
    tail = {n: inp[n][:1, cut:row_tokens] for n in names}
    s0 = None if inp["S0"] is None else inp["S0"][:1]
    _, S_cut = kda_oracle.forward(*(head[n] for n in names), S0=s0)
    o_true, _ = kda_oracle.forward(*(tail[n] for n in names), S0=S_cut)
    o_zero, _ = kda_oracle.forward(*(tail[n] for n in names), S0=None)
    moved = rel_err(o_zero[:, -span:], o_true[:, -span:])
    say(f"    dropping the state {3 * span} tokens before the end moves the last {span} outputs by "
        f"{moved:.3f} of RMS")
    assert moved > 0.1


@pytest.mark.parametrize("B,T,H,d,lengths", [
    (1, 16384, 2, 128, None),                        # 16 ranges of 16 chunks
    (2, 8192, 2, 64, None),
    (1, 0, 2, 128, [9000, 0, 7000, 1, 3072]),
])
def test_chunk_ranges_with_long_memory(B, T, H, d, lengths):
    inp = _long_memory_inputs(B, T, H, d, seed=1130 + d + (T or 1), lengths=lengths)
    assert _ranged(B, T, H, d, lengths)
    _assert_long_memory(inp, T if lengths is None else lengths[0])
    check(inp, 64, TOL[torch.bfloat16], label=f"long memory B{B} T{T} H{H} d{d} lengths={lengths}")


@pytest.mark.timeout(900)
def test_long_context_shape_with_long_memory_every_head():
    """B1 H32 T65536 (8 ranges of 128 chunks per head) with alpha = sigmoid(N(10, 1))
    and beta scaled by 0.01: a range's start state still moves the outputs two
    ranges (16,384 tokens) later; all 32 heads against the oracle."""
    say("[case] long-context shape, long memory: generating inputs")
    inp = _long_memory_inputs(1, 65536, 32, 128, seed=1150, alpha_mu=10.0, beta_scale=0.01)
    assert _ranged(1, 65536, 32, 128)
    _assert_long_memory(inp, 65536, span=8192)
    eo, es = whole_prefill_parity(inp, 64, 16, "long-context shape, long memory")
    assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16], (eo, es)


@pytest.mark.parametrize("every", [1024, 1536])
def test_chunk_ranges_with_long_memory_checkpoints(every):
    # ranges of 1,024 tokens: checkpoints on every range boundary, or on every
    # other one and mid-range
    inp = _long_memory_inputs(1, 16384, 2, 128, seed=1142)
    assert _ranged(1, 16384, 2, 128)
    _ckpt_check(inp, 64, every, 16384 // every, TOL[torch.bfloat16], f"long memory B1 T16384 H2 every {every}")


def test_chunk_ranges_with_long_memory_gated():
    inp = _long_memory_inputs(1, 16384, 2, 128, seed=1140)
    assert _ranged(1, 16384, 2, 128)
    _gate_case(inp, 64, TOL[torch.bfloat16], "long memory B1 T16384 H2")


def test_chunk_ranges_with_long_memory_windowed():
    # windows of about 5,000 tokens, each cut into ranges, resume from the
    # state the window before left
    inp = _long_memory_inputs(1, 16384, 2, 128, seed=1141)
    ws_bytes = _quote(1, 5000, 2, 128, 128, torch.bfloat16)
    og, Sg = _windowed(inp, ws_bytes)
    oo, So = oracle_prefill(inp)
    eo, es = rel_err(og, oo), rel_err(Sg, So)
    say(f"[case] long memory windowed: err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[torch.bfloat16] and es < TOL[torch.bfloat16]


def test_chunk_range_scan_dk64_packed_with_checkpoints():
    inp = workloads.make_inputs(1, 0, 3, 64, 64, torch.bfloat16, s0_std=0.02, seed=1125, lengths=[5000, 1, 4096])
    assert _ranged(1, 0, 3, 64, [5000, 1, 4096])
    _ckpt_check(inp, 64, 512, 10, TOL[torch.bfloat16], "ranges dk64 packed [5000, 1, 4096]")


def test_chunk_range_scan_resume_equals_one_pass():
    inp = workloads.make_inputs(1, 8192, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=1112)
    o_full, S_full = gpu_prefill(inp, 64)
    cut = 5000
    first = {k: (v[:, :cut].contiguous() if k in ("q", "k", "v", "alpha", "beta") else v) for k, v in inp.items()}
    o1, S1 = gpu_prefill(first, 64)
    second = {k: (v[:, cut:].contiguous() if k in ("q", "k", "v", "alpha", "beta") else v) for k, v in inp.items()}
    second["S0"] = torch.from_numpy(S1)
    o2, S2 = gpu_prefill(second, 64)
    assert rel_err(np.concatenate([o1, o2], axis=1), o_full) < 2e-2
    assert rel_err(S2, S_full) < 2e-2


# --- bounded-memory prefill (kda_chunk_fwd_windowed) --------------------------------
# Whole sequences are grouped while their workspace fits; longer ones run in
# windows of whole chunks that resume from the state the window before left.

def _quote(B, T, H, dk, dv, dtype, lengths=None):
    """kda_chunk_fwd_workspace_size of a call of that shape."""
    Tq = T if lengths is None else sum(lengths)
    q = torch.empty(B, Tq, H, dk, dtype=dtype, device="cuda")
    v = torch.empty(B, Tq, H, dv, dtype=dtype, device="cuda")
    cu = None if lengths is None else torch.zeros(len(lengths) + 1, dtype=torch.int32, device="cuda")
    return kda.workspace_size(q, v, cu)


def _windowed(inp, ws_bytes, chunk=64):
    d = to_dev(inp)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    o, S = kda.chunk_fwd_windowed(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ws, d["S0"], d["cu_seqlens"],
                                  chunk_size=chunk, o_dtype=torch.float32)
    torch.cuda.synchronize()
    return o.cpu().numpy(), S.cpu().numpy()


@pytest.mark.parametrize("B,T,H,d,dtype,lengths,budget", [
    (1, 5000, 2, 128, torch.bfloat16, None, 1500),                          # one sequence in 4 windows
    (1, 0, 3, 64, torch.bfloat16, [0, 300, 4000, 17, 0, 900, 2500], 1024),  # groups and windows
    (3, 700, 2, 128, torch.float32, None, 700),                             # one row per call
    (1, 0, 1, 32, torch.bfloat16, [0, 100, 0, 70], 0),                      # one chunk per call, empty ones alone
    (1, 20000, 2, 128, torch.bfloat16, None, 9000),                         # windows that take chunk ranges
])
def test_windowed_matches_oracle(B, T, H, d, dtype, lengths, budget):
    """``budget``: the workspace quote of one row of that many tokens, or (0) room
    for one chunk of one sequence and no more (one (chunk, head) block more than the
    status word; an empty sequence's own packed call would need two blocks)."""
    inp = workloads.make_inputs(B, T, H, d, d, dtype, s0_std=0.02, seed=1300 + d + H, lengths=lengths)
    if budget:
        ws_bytes = _quote(1, budget, H, d, d, dtype)
    else:
        ws_bytes = _quote(1, 128, H, d, d, dtype) - _quote(1, 64, H, d, d, dtype) + 512
    full = _quote(B, T, H, d, d, dtype, lengths)
    assert ws_bytes < full
    say(f"[case] windowed B{B} T{T} H{H} d{d} {dtype} lengths={lengths} workspace {ws_bytes} of {full}")
    og, Sg = _windowed(inp, ws_bytes)
    oo, So = oracle_prefill(inp)
    eo, es = rel_err(og, oo), rel_err(Sg, So)
    say(f"    err o={eo:.3e} S={es:.3e}")
    assert eo < TOL[dtype] and es < TOL[dtype]
    # and the same call in one piece
    o1, S1 = gpu_prefill(inp, 64)
    assert rel_err(og, o1) < TOL[dtype] and rel_err(Sg, S1) < TOL[dtype]


def test_windowed_packed_workload_matches_one_piece():
    """The packed variable-length workload (64 sequences up to 32,768 tokens, H16,
    nonzero initial states; device-drawn inputs) in a 2 GiB workspace against the
    one-piece call, whose parity with the oracle test_packed_varlen_resume_every_head
    checks on the CPU-drawn inputs."""
    d = workloads.device_inputs(workloads.PACKED_VARLEN_RESUME, torch.device("cuda"))
    say(f"[case] windowed packed workload {tuple(d['q'].shape)} in 2 GiB")
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    o1, S1 = kda.chunk_fwd(*args, d["S0"], d["cu_seqlens"], chunk_size=64, o_dtype=torch.float32)
    ws = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    assert ws.numel() < kda.workspace_size(d["q"], d["v"], d["cu_seqlens"]) // 8
    ow, Sw = kda.chunk_fwd_windowed(*args, ws, d["S0"], d["cu_seqlens"], chunk_size=64, o_dtype=torch.float32)
    torch.cuda.synchronize()
    eo = WholeTensorError()
    es = WholeTensorError()
    for h in range(o1.shape[2]):
        eo.add(ow[:, :, h].cpu().numpy(), o1[:, :, h].cpu().numpy())
        es.add(Sw[:, h].cpu().numpy(), S1[:, h].cpu().numpy())
    say(f"    windowed vs one piece: o={eo.value():.3e} S={es.value():.3e}")
    assert eo.value() < TOL[torch.bfloat16] and es.value() < TOL[torch.bfloat16]


@pytest.mark.parametrize("seed", range(8))
def test_windowed_random_plans(seed):
    """Seeded random bounded-workspace calls: packed (with empty sequences) or
    fixed-length, random heads, dims and dtype, a random subset of the options
    (gate, fused inputs, scalar decay, floor, checkpoints) and a random
    workspace budget, against the oracle and the one-piece call."""
    g = torch.Generator().manual_seed(8000 + seed)
    ri = lambda lo, hi: int(torch.randint(lo, hi, (1,), generator=g))
    H, d = ri(1, 4), [64, 128][ri(0, 2)]
    dtype = [torch.bfloat16, torch.float32][ri(0, 2)]
    opts = {}
    if ri(0, 2):
        opts["fuse_inputs"] = True
    if ri(0, 3) == 0:
        opts["alpha_scalar"] = True
    if ri(0, 3) == 0:
        opts["decay_floor"] = 0.5
    gated = bool(ri(0, 2))
    every = [0, 64, 128, 256][ri(0, 4)]
    if ri(0, 2):
        lens = [0 if ri(0, 5) == 0 else ri(1, 2500) for _ in range(ri(1, 7))]
        B, T = 1, 0
    else:
        lens, B, T = None, ri(1, 4), ri(1, 2500)
    n = B if lens is None else len(lens)
    inp = _prefill_opts_inputs(B, T, H, d, d, dtype, seed=8100 + seed, lengths=lens, **opts)
    extra = {}
    if gated:
        extra = {"gate": torch.randn(inp["v"].shape, generator=g).to(dtype), "norm_weight": torch.rand(d, generator=g) + 0.5,
                 "norm_eps": 1e-5}
    budget = max(ri(64, 3000), 2 * every)
    ws_bytes = _quote(1, budget, H, d, d, dtype)
    mx = ri(1, 12)
    say(f"[case] windowed random seed {seed}: B{B} T{T} lengths={lens} H{H} d{d} {dtype} opts={opts} "
        f"gated={gated} every={every} max={mx} budget {budget} tokens ({ws_bytes} B)")
    dd = to_dev(inp)
    dx = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in extra.items()}
    ck = torch.full((n, mx, H, d, d), float("nan"), device="cuda") if every else None
    ck1 = torch.full((n, mx, H, d, d), float("nan"), device="cuda") if every else None
    args = (dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ow, Sw = kda.chunk_fwd_windowed(*args, ws, dd["S0"], dd["cu_seqlens"], o_dtype=torch.float32, checkpoints=ck,
                                    ckpt_every=every, **opts, **dx)
    o1, S1 = kda.chunk_fwd(*args, dd["S0"], dd["cu_seqlens"], o_dtype=torch.float32, checkpoints=ck1,
                           ckpt_every=every, **opts, **dx)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"]
    res = kda_oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                             cu_seqlens=None if cu is None else cu.to(torch.int64), ckpt_every=every, max_ckpts=mx,
                             return_ckpt=bool(every), **opts, **extra)
    tol = TOL[dtype]
    eo, es = rel_err(ow.cpu().numpy(), res[0]), rel_err(Sw.cpu().numpy(), res[1])
    eo1, es1 = rel_err(ow.cpu().numpy(), o1.cpu().numpy()), rel_err(Sw.cpu().numpy(), S1.cpu().numpy())
    say(f"    vs oracle o={eo:.3e} S={es:.3e}; vs one piece o={eo1:.3e} S={es1:.3e}")
    assert eo < tol and es < tol and eo1 < tol and es1 < tol
    if every:
        cko, ckg = res[2], ck.cpu().numpy()
        written = ~np.isnan(cko).all(axis=(2, 3, 4))
        assert np.array_equal(~np.isnan(ckg).all(axis=(2, 3, 4)), written)
        if written.any():
            worst = max(rel_err(ckg[a, b], cko[a, b]) for a, b in zip(*np.nonzero(written)))
            say(f"    {int(written.sum())} checkpoints: {worst:.3e}")
            assert worst < tol


@pytest.mark.timeout(600)
def test_windowed_gated_packed_workload():
    """The packed workload (64 sequences, H16, S0 != 0) with the output norm and
    gate in a 2 GiB workspace: groups of a few sequences take one-slice
    workgroups and the epilogue, whose scratch rows start at the group's first
    token (up to ~10^6 tokens into the pack).  Against the one-piece gated call
    (whole rows) everywhere, and against the oracle on the first, a middle and
    the last sequence, every head."""
    d = workloads.device_inputs(workloads.PACKED_VARLEN_RESUME, torch.device("cuda"))
    g = torch.Generator(device="cuda").manual_seed(1330)
    gate = torch.randn(d["v"].shape, generator=g, device="cuda").to(torch.bfloat16)
    wn = torch.rand(d["v"].shape[-1], generator=g, device="cuda") + 0.5
    opts = {"gate": gate, "norm_weight": wn, "norm_eps": 1e-5}
    say(f"[case] windowed gated packed workload {tuple(d['q'].shape)} in 2 GiB")
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    o1, S1 = kda.chunk_fwd(*args, d["S0"], d["cu_seqlens"], o_dtype=torch.float32, **opts)
    ws = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    ow, Sw = kda.chunk_fwd_windowed(*args, ws, d["S0"], d["cu_seqlens"], o_dtype=torch.float32, **opts)
    torch.cuda.synchronize()
    del ws
    eo, es = WholeTensorError(), WholeTensorError()
    for h in range(o1.shape[2]):
        eo.add(ow[:, :, h].cpu().numpy(), o1[:, :, h].cpu().numpy())
        es.add(Sw[:, h].cpu().numpy(), S1[:, h].cpu().numpy())
    say(f"    windowed vs one piece: o={eo.value():.3e} S={es.value():.3e}")
    assert eo.value() < TOL[torch.bfloat16] and es.value() < TOL[torch.bfloat16]
    cu = d["cu_seqlens"].cpu().tolist()
    n_seq = len(cu) - 1
    for n in (0, n_seq // 2, n_seq - 1):
        t0, t1 = cu[n], cu[n + 1]
        sl = {k: d[k][:, t0:t1].cpu() for k in ("q", "k", "v", "alpha", "beta")}
        oo, So = kda_oracle.forward(sl["q"], sl["k"], sl["v"], sl["alpha"], sl["beta"], S0=d["S0"][n:n + 1].cpu(),
                                    gate=gate[:, t0:t1].cpu(), norm_weight=wn.cpu(), norm_eps=1e-5)
        e1, e2 = rel_err(ow[:, t0:t1].cpu().numpy(), oo), rel_err(Sw[n:n + 1].cpu().numpy(), So)
        say(f"    sequence {n} ({t1 - t0} tokens, from token {t0}) vs oracle: o={e1:.3e} S={e2:.3e}")
        assert e1 < TOL[torch.bfloat16] and e2 < TOL[torch.bfloat16]


def test_windowed_in_place_state():
    inp = workloads.make_inputs(1, 3000, 2, 64, 64, torch.bfloat16, s0_std=0.02, seed=1310)
    d = to_dev(inp)
    S = d["S0"].clone()
    ws = torch.empty(_quote(1, 640, 2, 64, 64, torch.bfloat16), dtype=torch.uint8, device="cuda")
    o, S_out = kda.chunk_fwd_windowed(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ws, S, None, final_state=S,
                                      o_dtype=torch.float32)
    assert S_out.data_ptr() == S.data_ptr()
    oo, So = oracle_prefill(inp)
    assert rel_err(o.cpu().numpy(), oo) < TOL[torch.bfloat16] and rel_err(S.cpu().numpy(), So) < TOL[torch.bfloat16]


def test_windowed_reports_a_range_error_of_an_early_window():
    """q past the fp16 range in the first window only: that window's outputs are not
    finite, the later windows' are, and the call still reports KDA_ERR_RANGE."""
    inp = workloads.make_inputs(1, 1024, 2, 128, 128, torch.bfloat16, s0_std=0.02, seed=1311)
    inp["q"][:, :64] = (inp["q"][:, :64].float() * 1e7).to(torch.bfloat16)
    d = to_dev(inp)
    ws = torch.empty(_quote(1, 256, 2, 128, 128, torch.bfloat16), dtype=torch.uint8, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.chunk_fwd_windowed(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ws, d["S0"], None)
    assert e.value.status == kda.KDA_ERR_RANGE
    o, S = kda.chunk_fwd_windowed(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ws, d["S0"], None,
                                  check_range=False)
    assert torch.isfinite(S).all() and torch.isfinite(o[:, 256:].float()).all()


# kda_chunk_fwd_windowed_ex: the options in bounded memory.  Each call of the
# split takes its tokens' rows of gate and alpha; with checkpoints the windows
# hold whole intervals and write into their sequence's slots.

WINDOWED_OPTS = [
    # (B, T, lengths, dk, dv, dtype, budget tokens, options, ckpt_every, max_ckpts, gated)
    (1, 0, [0, 300, 2000, 17, 900], 128, 128, torch.bfloat16, 700,
     {"fuse_inputs": True, "alpha_scalar": True, "decay_floor": 0.5}, 0, 0, True),
    (1, 3000, None, 128, 64, torch.bfloat16, 600, {}, 256, 8, False),        # slots run out at token 2048
    (1, 0, [100, 1500, 300, 0, 700], 64, 64, torch.bfloat16, 500, {"fuse_inputs": True}, 128, 6, True),
    (3, 700, None, 128, 128, torch.float32, 700, {"alpha_scalar": True}, 64, 12, True),
    # windows of 8,192 tokens that take chunk ranges and the gated ranged walk
    (1, 20000, None, 128, 128, torch.bfloat16, 9000, {"fuse_inputs": True}, 4096, 4, True),
]


@pytest.mark.parametrize("B,T,lengths,dk,dv,dtype,budget,opts,every,mx,gated", WINDOWED_OPTS)
def test_windowed_with_options_matches_oracle(B, T, lengths, dk, dv, dtype, budget, opts, every, mx, gated):
    H = 2
    inp = _prefill_opts_inputs(B, T, H, dk, dv, dtype, seed=1320 + budget, lengths=lengths, **opts)
    n = B if lengths is None else len(lengths)
    g = torch.Generator().manual_seed(1321 + budget)
    extra = {}
    if gated:
        extra = {"gate": torch.randn(inp["v"].shape, generator=g).to(dtype),
                 "norm_weight": torch.rand(dv, generator=g) + 0.5, "norm_eps": 1e-5}
    ws_bytes = _quote(1, budget, H, dk, dv, dtype)
    assert ws_bytes < _quote(B, T, H, dk, dv, dtype, lengths)
    say(f"[case] windowed options B{B} T{T} lengths={lengths} dk{dk} dv{dv} {dtype} {opts} every={every} "
        f"max={mx} gated={gated} workspace {ws_bytes}")
    d = to_dev(inp)
    dev_extra = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in extra.items()}
    ck = ckw = None
    if every:
        ck = torch.full((n, mx, H, dk, dv), float("nan"), device="cuda")
        ckw = torch.full((n, mx, H, dk, dv), float("nan"), device="cuda")
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ow, Sw = kda.chunk_fwd_windowed(*args, ws, d["S0"], d["cu_seqlens"], o_dtype=torch.float32, checkpoints=ckw,
                                    ckpt_every=every, **opts, **dev_extra)
    o1, S1 = kda.chunk_fwd(*args, d["S0"], d["cu_seqlens"], o_dtype=torch.float32, checkpoints=ck,
                           ckpt_every=every, **opts, **dev_extra)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"]
    res = kda_oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                             cu_seqlens=None if cu is None else cu.to(torch.int64), ckpt_every=every,
                             max_ckpts=mx, return_ckpt=bool(every), **opts, **extra)
    oo, So = res[0], res[1]
    tol = TOL[dtype]
    eo, es = rel_err(ow.cpu().numpy(), oo), rel_err(Sw.cpu().numpy(), So)
    eo1, es1 = rel_err(ow.cpu().numpy(), o1.cpu().numpy()), rel_err(Sw.cpu().numpy(), S1.cpu().numpy())
    say(f"    vs oracle o={eo:.3e} S={es:.3e}; vs one piece o={eo1:.3e} S={es1:.3e} (tol {tol})")
    assert eo < tol and es < tol and eo1 < tol and es1 < tol
    if every:
        cko = res[2]
        ckg, ck1 = ckw.cpu().numpy(), ck.cpu().numpy()
        written = ~np.isnan(cko).all(axis=(2, 3, 4))
        assert written.any()
        assert np.array_equal(~np.isnan(ckg).all(axis=(2, 3, 4)), written)   # the same slots, the rest untouched
        worst = max(rel_err(ckg[a, b], cko[a, b]) for a, b in zip(*np.nonzero(written)))
        worst1 = max(rel_err(ckg[a, b], ck1[a, b]) for a, b in zip(*np.nonzero(written)))
        say(f"    {int(written.sum())} checkpoints: vs oracle {worst:.3e}, vs one piece {worst1:.3e}")
        assert worst < tol and worst1 < tol
