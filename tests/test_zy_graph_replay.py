"""The prefill and decode calls captured in HIP graphs (torch.cuda.graph on a
side stream) and replayed: every replay equals the eager call bit for bit,
with other eager work on the default stream between the replays.  The calls
launch only kernels on the caller's stream (no memset, no host synchronisation,
no allocation inside the captured region), which is what capture needs.
"""
import pytest
import torch

import linear_attention_sequence_gated_amd as kda
import workloads

pytestmark = pytest.mark.gpu


def _inputs(seed, T=300, H=2, d=128, lengths=None):
    inp = workloads.make_inputs(1, T, H, d, d, torch.bfloat16, s0_std=0.02, seed=seed, lengths=lengths)
    return {k: (v.cuda() if v is not None else None) for k, v in inp.items()}


def _other_eager_work(seed):
    """An unrelated eager prefill on the default stream between replays."""
    e = _inputs(seed, T=200)
    kda.chunk_fwd(e["q"], e["k"], e["v"], e["alpha"], e["beta"], e["S0"], None, o_dtype=torch.float32)


@pytest.mark.parametrize("lengths", [None, [0, 130, 64, 1, 105]])
def test_prefill_graph_replays_equal_eager(lengths):
    d = _inputs(1400, lengths=lengths)
    print(f"[case] prefill graph q={tuple(d['q'].shape)} lengths={lengths}", flush=True)
    s = torch.cuda.Stream()
    o = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
    S = torch.empty_like(d["S0"])
    pre = kda.Prefill(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], d["cu_seqlens"], chunk_size=64,
                      o=o, final_state=S, o_dtype=torch.float32, stream=s)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pre.run()                      # eager, on the capture stream
    s.synchronize()
    o_ref, S_ref = o.clone(), S.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pre.run()
    for i in range(4):
        o.fill_(float("nan"))
        S.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), f"replay {i}"
        _other_eager_work(1500 + i)
        torch.cuda.synchronize()
    assert pre.status() == 0


def test_noalloc_prefill_graph_replays_equal_eager():
    d = _inputs(1401, T=700)
    print(f"[case] noalloc prefill graph q={tuple(d['q'].shape)}", flush=True)
    o = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
    S = torch.empty_like(d["S0"])
    s = torch.cuda.Stream()
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"], None)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kda.chunk_fwd_noalloc(*args, o=o, final_state=S, o_dtype=torch.float32, stream=s)
    s.synchronize()
    o_ref, S_ref = o.clone(), S.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        kda.chunk_fwd_noalloc(*args, o=o, final_state=S, o_dtype=torch.float32, stream=s)
    for i in range(4):
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), f"replay {i}"
        _other_eager_work(1600 + i)
        torch.cuda.synchronize()


def test_decode_steps_graph_replays_equal_eager():
    """Four in-place decode steps in one graph."""
    n, H, d, steps = 16, 4, 128, 4
    dec = workloads.make_inputs(steps, n, H, d, d, torch.bfloat16, seed=1402)
    x = {k: (v.cuda() if v is not None else None) for k, v in dec.items()}
    S0 = (torch.randn(n, H, d, d, generator=torch.Generator().manual_seed(3)) * 0.02).cuda()
    print(f"[case] decode graph n={n} H={H} steps={steps}", flush=True)
    state = S0.clone()
    outs = [torch.empty(n, H, d, dtype=torch.float32, device="cuda") for _ in range(steps)]
    s = torch.cuda.Stream()

    def run():
        for t in range(steps):
            kda.decode_step(x["q"][t], x["k"][t], x["v"][t], x["alpha"][t], x["beta"][t], state, o=outs[t],
                            o_dtype=torch.float32)

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    s.synchronize()
    ref_o = [t.clone() for t in outs]
    ref_S = state.clone()
    state.copy_(S0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    for i in range(4):
        state.copy_(S0)
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref_o)) and torch.equal(state, ref_S), f"replay {i}"
        _other_eager_work(1700 + i)
        torch.cuda.synchronize()


def test_windowed_gated_prefill_graph_replays_equal_eager():
    """kda_chunk_fwd_windowed_ex (output norm and gate) in a workspace that
    holds a few chunks: packed groups and windows that resume from the state,
    with the status folds between the calls, all in one graph."""
    lengths = [0, 300, 1000, 17, 200]
    d = _inputs(1403, lengths=lengths)
    g0 = torch.Generator(device="cuda").manual_seed(4)
    gate = torch.randn(d["v"].shape, generator=g0, device="cuda").to(torch.bfloat16)
    wn = torch.rand(d["v"].shape[-1], generator=g0, device="cuda") + 0.5
    cu_host = d["cu_seqlens"].cpu()    # the host copy, made before the capture
    q1 = torch.empty(1, 400, 2, 128, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(kda.workspace_size(q1, q1), dtype=torch.uint8, device="cuda")
    o = torch.empty(d["v"].shape, dtype=torch.float32, device="cuda")
    S = torch.empty_like(d["S0"])
    print(f"[case] windowed gated prefill graph lengths={lengths} workspace {ws.numel()}", flush=True)
    s = torch.cuda.Stream()

    def run():
        kda.chunk_fwd_windowed(d["q"], d["k"], d["v"], d["alpha"], d["beta"], ws, d["S0"], d["cu_seqlens"],
                               o=o, final_state=S, o_dtype=torch.float32, stream=s, check_range=False,
                               cu_seqlens_host=cu_host, gate=gate, norm_weight=wn, norm_eps=1e-5)

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    s.synchronize()
    o_ref, S_ref = o.clone(), S.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run()
    for i in range(4):
        o.fill_(float("nan"))
        S.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), f"replay {i}"
        _other_eager_work(1800 + i)
        torch.cuda.synchronize()
    assert kda.load().kda_chunk_fwd_status(ws.data_ptr(), None) == 0
