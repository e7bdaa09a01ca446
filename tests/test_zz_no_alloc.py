"""kda_chunk_fwd_noalloc (the allocation-free entry point) against kda_chunk_fwd.

Both run the same kernels on the same workspace layout, so their outputs must
be identical; each is also within the parity bound of the fp64 oracle.  Two
calls in a row, the second with a smaller input, check that the scratch the
library keeps between calls carries nothing from one call into the next.
"""
import pytest
import torch

import linear_attention_sequence_gated_amd as kda
import workloads
from oracle import kda_oracle
from parity_measure import rel_err

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def _case(B, T, H, dk, dv, dtype, seed, lengths=None):
    inp = workloads.make_inputs(B, T, H, dk, dv, dtype, s0_std=0.02, seed=seed, lengths=lengths)
    d = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    return inp, d


def _compare(inp, d, chunk):
    print(f"[case] noalloc q={tuple(inp['q'].shape)} {inp['q'].dtype} chunk={chunk}", flush=True)
    o_ref, s_ref = kda.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"],
                                 chunk_size=chunk, o_dtype=torch.float32)
    o_na = torch.full_like(o_ref, float("nan"))
    s_na = torch.full_like(s_ref, float("nan"))
    kda.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"], o=o_na,
                          final_state=s_na, chunk_size=chunk, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref) and torch.equal(s_na, s_ref)
    cu = inp["cu_seqlens"]
    oo, so = kda_oracle.forward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                                cu_seqlens=None if cu is None else cu.to(torch.int64))
    tol = TOL[inp["q"].dtype]
    eo, es = rel_err(o_na.cpu().numpy(), oo), rel_err(s_na.cpu().numpy(), so)
    print(f"    err o={eo:.3e} S={es:.3e} (tol {tol})", flush=True)
    assert eo < tol and es < tol


def test_noalloc_matches_chunk_fwd_two_calls_second_smaller():
    inp, d = _case(2, 700, 4, 128, 128, torch.bfloat16, seed=801)
    _compare(inp, d, 64)
    inp, d = _case(1, 0, 2, 128, 64, torch.bfloat16, seed=802, lengths=[5, 0, 130, 64])
    _compare(inp, d, 64)


def test_noalloc_with_chunk_ranges():
    # few long sequences: the range maps, the scanned start states and the
    # ranged walk all live in the library's scratch
    inp, d = _case(1, 3072, 4, 128, 128, torch.bfloat16, seed=804)
    plan = kda.chunk_plan(d["q"], d["v"])
    assert plan["range_chunks"] > 0, plan
    assert kda.workspace_size(d["q"], d["v"]) <= kda._lib.NOALLOC_SCRATCH_BYTES
    _compare(inp, d, 64)


def test_noalloc_fp32_and_rejects_oversize():
    inp, d = _case(1, 150, 2, 64, 32, torch.float32, seed=803)
    _compare(inp, d, 32)
    # a call whose workspace exceeds the scratch is refused before any launch
    big = torch.empty((1, 65536, 32, 128), dtype=torch.bfloat16, device="cuda")
    al = torch.empty((1, 65536, 32, 128), dtype=torch.float32, device="cuda")
    be = torch.empty((1, 65536, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.chunk_fwd_noalloc(big, big, big, al, be)
    assert e.value.status == 3   # KDA_ERR_WORKSPACE
