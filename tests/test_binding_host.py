"""Host-side checks of the Python binding and of the parity measure (no GPU).

The binding must reject a malformed tensor argument with ValueError before it
allocates anything or calls the library: an undersized, strided or host
tensor handed to a kernel would be read or written out of bounds on the
device.  Tensors on the "meta" device stand in for device tensors here (they
carry shape, dtype and strides but no memory), and torch.empty and the
library loader are replaced by functions that fail the test if reached.
"""
import numpy as np
import pytest
import torch

from linear_attention_sequence_gated_amd import _lib
from parity_measure import WholeTensorError, rel_err

B, T, H, DK, DV = 1, 96, 2, 64, 32


def _meta(*shape, dtype=torch.bfloat16):
    return torch.empty(*shape, dtype=dtype, device="meta")


@pytest.fixture
def guarded(monkeypatch):
    """Meta tensors count as device tensors; any allocation or library call fails."""
    monkeypatch.setattr(_lib, "_on_device", lambda t: t.device.type == "meta")

    def reached(*a, **k):
        raise AssertionError("the binding allocated or called the library before rejecting the call")
    yield lambda: (monkeypatch.setattr(_lib.torch, "empty", reached), monkeypatch.setattr(_lib, "load", reached))


def _prefill_args(n=B, lengths=None):
    args = dict(q=_meta(B, T, H, DK), k=_meta(B, T, H, DK), v=_meta(B, T, H, DV),
                alpha=_meta(B, T, H, DK, dtype=torch.float32), beta=_meta(B, T, H, dtype=torch.float32))
    return args


PREFILL_BAD = {
    "final_state too small": dict(final_state=_meta(B, H, DK, DV - 1, dtype=torch.float32)),
    "final_state fp16": dict(final_state=_meta(B, H, DK, DV, dtype=torch.float16)),
    "final_state strided": dict(final_state=_meta(B, H, DV, DK, dtype=torch.float32).transpose(2, 3)),
    "final_state on the host": dict(final_state=torch.zeros(B, H, DK, DV)),
    "initial_state on the host": dict(initial_state=torch.zeros(B, H, DK, DV)),
    "initial_state wrong shape": dict(initial_state=_meta(B, H + 1, DK, DV, dtype=torch.float32)),
    "o on the host": dict(o=torch.zeros(B, T, H, DV, dtype=torch.bfloat16)),
    "o wrong dtype": dict(o=_meta(B, T, H, DV, dtype=torch.float16)),
    "o strided": dict(o=_meta(B, T, DV, H).transpose(2, 3)),
    "gate wrong dtype": dict(gate=_meta(B, T, H, DV, dtype=torch.float32)),
    "norm_weight strided": dict(gate=_meta(B, T, H, DV), norm_weight=_meta(2 * DV, dtype=torch.float32)[::2]),
    "norm_weight on the host": dict(gate=_meta(B, T, H, DV), norm_weight=torch.ones(DV)),
    "cu_seqlens int64": dict(cu_seqlens=_meta(3, dtype=torch.int64)),
    "cu_seqlens strided": dict(cu_seqlens=_meta(6, dtype=torch.int32)[::2]),
    "cu_seqlens on the host": dict(cu_seqlens=torch.tensor([0, 40, 96], dtype=torch.int32)),
}


@pytest.mark.parametrize("case", sorted(PREFILL_BAD))
def test_prefill_rejects_bad_tensor(guarded, case):
    args = _prefill_args()
    guarded()
    with pytest.raises(ValueError, match=rf"^{case.split()[0]} must"):   # rejected for that tensor
        _lib.Prefill(**args, **PREFILL_BAD[case])


WINDOWED_BAD = {
    "workspace on the host": dict(workspace=torch.zeros(1 << 10, dtype=torch.uint8)),
    "final_state too small": dict(final_state=_meta(B, H, DK, DV - 1, dtype=torch.float32)),
    "initial_state on the host": dict(initial_state=torch.zeros(B, H, DK, DV)),
    "cu_seqlens_host on the device": dict(cu_seqlens=_meta(3, dtype=torch.int32),
                                          cu_seqlens_host=_meta(3, dtype=torch.int32)),
    "cu_seqlens_host int64": dict(cu_seqlens=_meta(3, dtype=torch.int32), cu_seqlens_host=torch.tensor([0, 40, 96])),
    "cu_seqlens_host short": dict(cu_seqlens=_meta(3, dtype=torch.int32),
                                  cu_seqlens_host=torch.tensor([0, 96], dtype=torch.int32)),
    "cu_seqlens_host alone": dict(cu_seqlens_host=torch.tensor([0, 40, 96], dtype=torch.int32)),
    "gate wrong dtype": dict(gate=_meta(B, T, H, DV, dtype=torch.float32)),
    "norm_weight on the host": dict(gate=_meta(B, T, H, DV), norm_weight=torch.ones(DV)),
    "checkpoints wrong shape": dict(checkpoints=_meta(B, 2, H, DK, DV + 1, dtype=torch.float32), ckpt_every=64),
    "alpha per channel with alpha_scalar": dict(alpha_scalar=True),
}


@pytest.mark.parametrize("case", sorted(WINDOWED_BAD))
def test_windowed_rejects_bad_tensor(guarded, case):
    args = _prefill_args()
    args["workspace"] = _meta(1 << 20, dtype=torch.uint8)
    args.update(WINDOWED_BAD[case])
    guarded()
    with pytest.raises(ValueError, match=rf"^{case.split()[0]} must"):
        _lib.chunk_fwd_windowed(**args)


def _decode_args():
    n = 3
    return dict(q=_meta(n, H, DK), k=_meta(n, H, DK), v=_meta(n, H, DV), alpha=_meta(n, H, DK, dtype=torch.float32),
                beta=_meta(n, H, dtype=torch.float32), state=_meta(n, H, DK, DV, dtype=torch.float32))


DECODE_BAD = {
    "o on the host": dict(o=torch.zeros(3, H, DV, dtype=torch.bfloat16)),
    "o wrong shape": dict(o=_meta(3, H, DV + 1)),
    "state on the host": dict(state=torch.zeros(3, H, DK, DV)),
    "state strided": dict(state=_meta(3, H, DV, DK, dtype=torch.float32).transpose(2, 3)),
    "norm_weight strided": dict(gate=_meta(3, H, DV), norm_weight=_meta(2 * DV, dtype=torch.float32)[::2]),
    "state_slots strided": dict(state=_meta(5, H, DK, DV, dtype=torch.float32),
                                state_slots=_meta(6, dtype=torch.int32)[::2]),
    "state_slots on the host": dict(state=_meta(5, H, DK, DV, dtype=torch.float32),
                                    state_slots=torch.tensor([4, 0, 2], dtype=torch.int32)),
}


@pytest.mark.parametrize("case", sorted(DECODE_BAD))
def test_decode_rejects_bad_tensor(guarded, case):
    args = _decode_args()
    args.update(DECODE_BAD[case])
    guarded()
    with pytest.raises(ValueError, match=rf"^{case.split()[0]}"):
        _lib.decode_step(**args)


def test_whole_tensor_error_equals_rel_err_of_the_concatenation():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((7, 300, 5))
    gpu = ref + 1e-3 * rng.standard_normal(ref.shape)
    gpu[3, 17, 2] += 0.5                     # the largest deviation sits in one piece
    acc = WholeTensorError()
    for h in range(5):                       # pieces along the last axis, in small row blocks
        acc.add(gpu[..., h], ref[..., h], rows=97)
    assert acc.value() == pytest.approx(rel_err(gpu, ref), rel=1e-12)
    assert acc.max_diff == pytest.approx(float(np.max(np.abs(gpu - ref))), rel=1e-12)


def test_whole_tensor_error_rejects_non_finite():
    with pytest.raises(AssertionError):
        WholeTensorError().add(np.array([1.0, np.inf]), np.array([1.0, 1.0]))


@pytest.mark.parametrize("opts", [dict(alpha_scalar=True), dict(decay_floor=0.5), dict(fuse_inputs=True)])
def test_split_phases_refuse_calls_with_options(monkeypatch, opts, guarded):
    """kda_chunk_fwd_intra / _inter take no options: a call object with options
    (here a per-token alpha, a floor, fused inputs) must not reach them, or its
    tensors would be read in the plain layout."""
    monkeypatch.setattr(_lib, "_on_device", lambda t: t.device.type == "meta")
    args = _prefill_args()
    if opts.get("alpha_scalar"):
        args["alpha"] = _meta(B, T, H, dtype=torch.float32)
    pre = _lib.Prefill(**args, **opts, stream=type("S", (), {"cuda_stream": 0})())   # no device here

    def reached(*a, **k):
        raise AssertionError("a split phase reached the library")
    monkeypatch.setattr(pre, "_lib", type("L", (), {"kda_chunk_fwd_intra": reached, "kda_chunk_fwd_inter": reached}))
    for phase in (pre.intra, pre.inter):
        with pytest.raises(ValueError, match="plain call only"):
            phase()
