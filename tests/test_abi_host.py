"""Host-side checks of libkda.so that need no GPU.

The library must load, export every function include/kda.h declares, and
reject invalid arguments with the documented status before anything is
launched (every call here is invalid, so none reaches a kernel).
"""
import ctypes
import os
import re

import pytest
import torch

import linear_attention_sequence_gated_amd as kda
from linear_attention_sequence_gated_amd._lib import ChunkOptions, ChunkParams, ChunkPlan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x10000)      # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10008)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from linear_attention_sequence_gated_amd import build
    if build.is_stale():
        build.build()
    return kda.load()


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert declared == sorted(kda.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(6):
        s = kda.status_string(code)
        assert s.startswith("KDA_")
    assert "unknown" in kda.status_string(99)


def _params(**kw):
    p = dict(batch=1, seqlen=128, num_seqs=1, num_heads=2, head_dim_k=128, head_dim_v=128,
             chunk_size=64, scale=1.0, qkv_dtype=1, o_dtype=1)
    p.update(kw)
    return ChunkParams(**p)


def _ws(lib, p):
    out = ctypes.c_size_t(0)
    st = lib.kda_chunk_fwd_workspace_size(ctypes.byref(p), ctypes.byref(out))
    return st, out.value


def test_workspace_size(lib):
    st, n1 = _ws(lib, _params())
    assert st == OK and n1 > 0
    st, n2 = _ws(lib, _params(seqlen=256))
    assert st == OK and n2 > n1                      # grows with T
    st, n3 = _ws(lib, _params(num_heads=4))
    assert st == OK and n3 > n2 - 1                  # grows with H
    st, n4 = _ws(lib, _params(batch=1, num_seqs=40, seqlen=128))
    assert st == OK and n4 > n1                      # packed worst case: one partial chunk per sequence
    assert _ws(lib, _params(head_dim_k=96))[0] == UNSUPPORTED
    assert _ws(lib, _params(chunk_size=128))[0] == UNSUPPORTED
    assert _ws(lib, _params(qkv_dtype=7))[0] == UNSUPPORTED
    assert _ws(lib, _params(o_dtype=3))[0] == UNSUPPORTED
    # fp32 operands with dk = 128 run 32-token chunks: the quote does not depend
    # on a requested 64
    assert _ws(lib, _params(qkv_dtype=0, chunk_size=64)) == _ws(lib, _params(qkv_dtype=0, chunk_size=32))
    assert _ws(lib, _params(num_heads=0))[0] == INVALID
    assert lib.kda_chunk_fwd_workspace_size(None, None) == INVALID


def _plan(lib, p, packed=0):
    out = ChunkPlan()
    st = lib.kda_chunk_fwd_plan(ctypes.byref(p), packed, ctypes.byref(out))
    return st, (out.chunk_size, out.whole_rows, out.range_chunks, out.max_ranges)


def test_plan(lib):
    """Chunk ranges for bf16 dk = dv in {64, 128} with fewer (sequence, head)
    pairs than compute units (256 assumed without a device) and at least three
    ranges of max(16, ceil(chunks * pairs / 256)) chunks per sequence."""
    if torch.cuda.device_count() > 0 and torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("expected values assume 256 compute units")
    # 32 heads of 1024 chunks: ranges of 1024 * 32 / 256 = 128 chunks, 8 per sequence
    assert _plan(lib, _params(seqlen=65536, num_heads=32)) == (OK, (64, 1, 128, 8))
    # 48 chunks make three 16-chunk ranges; 47 do not
    assert _plan(lib, _params(seqlen=3072, num_heads=4)) == (OK, (64, 1, 16, 3))
    assert _plan(lib, _params(seqlen=3008, num_heads=4)) == (OK, (64, 0, 0, 0))
    assert _plan(lib, _params(batch=2, num_seqs=2, seqlen=5000, num_heads=2, head_dim_k=64,
                              head_dim_v=64)) == (OK, (64, 1, 16, 10))
    # as many pairs as compute units: whole rows, no ranges
    assert _plan(lib, _params(seqlen=65536, num_heads=256)) == (OK, (64, 1, 0, 0))
    # fp32 operands (32-token chunks at dk = 128), dk != dv and 32-token chunks take no ranges
    assert _plan(lib, _params(seqlen=65536, qkv_dtype=0, o_dtype=0)) == (OK, (32, 0, 0, 0))
    assert _plan(lib, _params(seqlen=65536, head_dim_v=64)) == (OK, (64, 0, 0, 0))
    assert _plan(lib, _params(seqlen=65536, chunk_size=32)) == (OK, (32, 0, 0, 0))
    # packed, 20073 tokens in 5 sequences: at most 313 + 5 + 1 chunks per head,
    # 63 on average; ranges of 16, at most 319 / 16 + 5 + 1 of them
    assert _plan(lib, _params(num_seqs=5, seqlen=20073), packed=1) == (OK, (64, 1, 16, 25))
    assert _plan(lib, _params(batch=2, num_seqs=2, seqlen=20073), packed=1)[0] == INVALID
    assert _plan(lib, _params(head_dim_k=96))[0] == UNSUPPORTED
    assert lib.kda_chunk_fwd_plan(ctypes.byref(_params()), 0, None) == INVALID


def test_gated_workspace_adds_epilogue_scratch_only_for_one_slice_shapes(lib):
    """The epilogue's scratch (fp32 outputs and per-slice sums of squares) is
    quoted for gated calls only where they take one-slice workgroups."""
    if torch.cuda.device_count() > 0 and torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the layouts assume 256 compute units")
    gated = ChunkOptions(gate=FAKE.value)

    def quotes(**kw):
        p = _params(**kw)
        plain, gate = ctypes.c_size_t(0), ctypes.c_size_t(0)
        assert lib.kda_chunk_fwd_ex_workspace_size(ctypes.byref(p), None, ctypes.byref(plain)) == OK
        assert lib.kda_chunk_fwd_ex_workspace_size(ctypes.byref(p), ctypes.byref(gated), ctypes.byref(gate)) == OK
        return plain.value, gate.value

    T, H, dv = 2048, 4, 128   # 32 chunks over 4 pairs: one-slice workgroups in either layout
    plain, gate = quotes(seqlen=T, num_heads=H)
    scratch = -(-T * H * dv * 4 // 256) * 256 + -(-T * H * (dv // 16) * 4 // 256) * 256
    assert gate >= plain + scratch
    for kw in (dict(seqlen=65536, num_heads=32),     # chunk ranges
               dict(seqlen=256, num_heads=256)):     # whole rows
        plain, gate = quotes(**kw)
        assert gate == plain, kw


def _fwd(lib, p, q=FAKE, k=FAKE, v=FAKE, a=FAKE, b=FAKE, s0=None, cu=None, o=FAKE, sf=None,
         ws=None, wsb=0):
    return lib.kda_chunk_fwd(ctypes.byref(p) if p is not None else None, q, k, v, a, b, s0, cu, o,
                             sf, ws, ctypes.c_size_t(wsb), None)


def test_chunk_fwd_rejects_before_launch(lib):
    p = _params()
    _, need = _ws(lib, p)
    assert _fwd(lib, None) == INVALID
    assert _fwd(lib, p, q=None, ws=FAKE, wsb=need) == INVALID
    assert _fwd(lib, p, o=None, ws=FAKE, wsb=need) == INVALID
    assert _fwd(lib, p, q=MISALIGNED, ws=FAKE, wsb=need) == INVALID
    assert _fwd(lib, p, b=ctypes.c_void_p(0x10002), ws=FAKE, wsb=need) == INVALID
    assert _fwd(lib, p, ws=None, wsb=0) == WORKSPACE
    assert _fwd(lib, p, ws=FAKE, wsb=1) == WORKSPACE
    assert _fwd(lib, p, ws=ctypes.c_void_p(0x10010), wsb=need) == WORKSPACE   # not 256-aligned
    assert _fwd(lib, _params(head_dim_v=48), ws=FAKE, wsb=need) == UNSUPPORTED
    assert _fwd(lib, _params(num_seqs=2), ws=FAKE, wsb=need) == INVALID      # N != B without cu
    assert _fwd(lib, _params(batch=2, num_seqs=2), cu=FAKE, ws=FAKE, wsb=10 * need) == INVALID
    assert _fwd(lib, _params(scale=float("nan")), ws=FAKE, wsb=need) == INVALID
    # states that overlap without being the same buffer
    assert _fwd(lib, p, s0=ctypes.c_void_p(0x100000), sf=ctypes.c_void_p(0x100010), ws=FAKE,
                wsb=need) == INVALID


def _fwd_ex(lib, p, opt, sf=None, ws=FAKE, wsb=1 << 40):
    return lib.kda_chunk_fwd_ex(ctypes.byref(p), ctypes.byref(opt) if opt is not None else None, FAKE, FAKE,
                                FAKE, FAKE, FAKE, None, None, FAKE, sf, ws, ctypes.c_size_t(wsb), None)


def test_chunk_fwd_ex_rejects_bad_options_before_launch(lib):
    p = _params()
    ck = ctypes.c_void_p(0x200000)
    Opt = kda.ChunkOptions
    assert _fwd_ex(lib, p, Opt(checkpoints=ck.value, ckpt_every=100, max_ckpts=2)) == INVALID   # not a multiple of 64
    assert _fwd_ex(lib, p, Opt(checkpoints=ck.value, ckpt_every=-64, max_ckpts=2)) == INVALID
    assert _fwd_ex(lib, p, Opt(checkpoints=None, ckpt_every=64, max_ckpts=2)) == INVALID
    assert _fwd_ex(lib, p, Opt(checkpoints=ck.value, ckpt_every=64, max_ckpts=0)) == INVALID
    assert _fwd_ex(lib, p, Opt(checkpoints=0x200004, ckpt_every=64, max_ckpts=1)) == INVALID     # misaligned
    # checkpoints that overlap the final state
    assert _fwd_ex(lib, p, Opt(checkpoints=ck.value, ckpt_every=64, max_ckpts=1),
                   sf=ctypes.c_void_p(ck.value + 256)) == INVALID
    assert _fwd_ex(lib, p, Opt(decay_floor=-0.1)) == INVALID
    assert _fwd_ex(lib, p, Opt(decay_floor=float("nan"))) == INVALID
    assert _fwd_ex(lib, p, Opt(alpha_mode=2)) == INVALID
    assert _fwd_ex(lib, p, Opt(fuse_inputs=5)) == INVALID
    assert _fwd_ex(lib, p, Opt(norm_weight=0x300000)) == INVALID        # a norm weight needs a gate
    assert _fwd_ex(lib, p, Opt(gate=0x300001)) == INVALID                # misaligned gate
    assert _fwd_ex(lib, p, Opt(gate=0x300000, norm_eps=-1.0)) == INVALID


def test_decode_step_rejects_before_launch(lib):
    def call(n=4, h=2, dk=128, dv=128, scale=1.0, dt=1, odt=1, ptrs=None):
        ptrs = ptrs or [FAKE] * 8
        return lib.kda_decode_step(n, h, dk, dv, scale, dt, odt, *ptrs, None)
    assert call(n=0) == INVALID
    assert call(h=0) == INVALID
    assert call(dk=256) == UNSUPPORTED
    assert call(dv=24) == UNSUPPORTED
    assert call(dt=5) == UNSUPPORTED
    assert call(odt=-1) == UNSUPPORTED
    assert call(scale=float("nan")) == INVALID
    assert call(ptrs=[FAKE] * 5 + [None] + [FAKE] * 2) == INVALID       # state
    assert call(ptrs=[FAKE] * 5 + [MISALIGNED] + [FAKE] * 2) == INVALID  # state alignment


def test_decode_step_ex_rejects_bad_options_before_launch(lib):
    Opt = kda.DecodeOptions

    def call(opt, alpha=FAKE):
        return lib.kda_decode_step_ex(2, 2, 64, 64, 1.0, 1, 0, ctypes.byref(opt), FAKE, FAKE, FAKE, alpha, FAKE,
                                      FAKE, FAKE, None)
    assert call(Opt(decay_floor=-0.5)) == INVALID
    assert call(Opt(decay_floor=float("nan"))) == INVALID
    assert call(Opt(norm_eps=-1.0, gate=0x30000)) == INVALID
    assert call(Opt(alpha_mode=2)) == INVALID
    assert call(Opt(fuse_inputs=3)) == INVALID
    assert call(Opt(state_slots=0x30002)) == INVALID                 # misaligned slots
    assert call(Opt(state_slots=0x30000, pool_entries=-1)) == INVALID  # a pool of negative size
    assert call(Opt(norm_weight=0x30000)) == INVALID                 # a norm weight needs a gate
    assert call(Opt(), alpha=MISALIGNED) == INVALID                  # per-channel alpha: 16-byte aligned
    assert call(Opt(alpha_mode=1), alpha=ctypes.c_void_p(0x10003)) == INVALID


def test_noalloc_rejects_before_any_launch(lib):
    # the library-held scratch holds 64 MiB: a long-context shape is refused,
    # and bad parameters are refused as by kda_chunk_fwd, with no device call
    fn = lib.kda_chunk_fwd_noalloc
    args = [FAKE] * 9 + [None]
    big = _params(seqlen=65536, num_heads=32)
    assert fn(ctypes.byref(big), *args) == WORKSPACE
    assert fn(ctypes.byref(_params(head_dim_k=96)), *args) == UNSUPPORTED
    assert fn(ctypes.byref(_params(num_heads=0)), *args) == INVALID
    assert fn(None, *args) == INVALID


def test_status_query_rejects_bad_workspace(lib):
    assert lib.kda_chunk_fwd_status(None, None) == INVALID
    assert lib.kda_chunk_fwd_status(ctypes.c_void_p(0x10010), None) == INVALID   # not 256-byte aligned


def _windowed(lib, p, cu=None, cu_host=None, final=FAKE, init=None, ws=FAKE, ws_bytes=1 << 40, q=FAKE):
    return lib.kda_chunk_fwd_windowed(ctypes.byref(p), q, FAKE, FAKE, FAKE, FAKE, init, cu, cu_host, FAKE, final,
                                      ws, ws_bytes, None)


def test_windowed_rejects_bad_arguments_before_launching(lib):
    p = _params(seqlen=4096)
    assert _windowed(lib, p, final=None) == INVALID              # final_state carries the state
    assert _windowed(lib, p, final=MISALIGNED) == INVALID
    assert _windowed(lib, p, q=MISALIGNED) == INVALID
    assert _windowed(lib, p, init=MISALIGNED) == INVALID
    pk = _params(seqlen=100, num_seqs=2)
    good = (ctypes.c_int32 * 3)(0, 60, 100)
    assert _windowed(lib, pk, cu=FAKE) == INVALID                 # device cu_seqlens without its host copy
    assert _windowed(lib, pk, cu_host=good) == INVALID            # host copy without the device array
    assert _windowed(lib, pk, cu=FAKE, cu_host=(ctypes.c_int32 * 3)(0, 60, 99)) == INVALID    # cu[N] != T
    assert _windowed(lib, pk, cu=FAKE, cu_host=(ctypes.c_int32 * 3)(1, 60, 100)) == INVALID   # cu[0] != 0
    assert _windowed(lib, pk, cu=FAKE, cu_host=(ctypes.c_int32 * 3)(0, 110, 100)) == INVALID  # decreasing
    assert _windowed(lib, _params(batch=2, num_seqs=2, seqlen=50), cu=FAKE, cu_host=good) == INVALID
    assert _windowed(lib, p, ws=None) == WORKSPACE
    assert _windowed(lib, p, ws=MISALIGNED) == WORKSPACE
    # too small for one chunk of one sequence (one block alone is ~74 KB here)
    assert _windowed(lib, p, ws_bytes=4096) == WORKSPACE
    assert _windowed(lib, pk, cu=FAKE, cu_host=good, ws_bytes=4096) == WORKSPACE
    assert _windowed(lib, _params(head_dim_k=96)) == UNSUPPORTED


def _windowed_ex(lib, p, opt, ws_bytes=1 << 40, alpha=FAKE, final=FAKE):
    return lib.kda_chunk_fwd_windowed_ex(ctypes.byref(p), ctypes.byref(opt), FAKE, FAKE, FAKE, alpha, FAKE, None,
                                         None, None, FAKE, final, FAKE, ws_bytes, None)


def test_windowed_ex_rejects_bad_options_before_launching(lib):
    p = _params(seqlen=4096)
    Opt = kda.ChunkOptions
    ck = ctypes.c_void_p(0x200000)
    assert _windowed_ex(lib, p, Opt(checkpoints=ck.value, ckpt_every=100, max_ckpts=2)) == INVALID
    assert _windowed_ex(lib, p, Opt(checkpoints=ck.value, ckpt_every=64, max_ckpts=0)) == INVALID
    assert _windowed_ex(lib, p, Opt(checkpoints=ck.value, ckpt_every=64, max_ckpts=1),
                        final=ctypes.c_void_p(ck.value + 256)) == INVALID        # overlaps the states
    assert _windowed_ex(lib, p, Opt(gate=0x10001)) == INVALID                    # misaligned gate
    assert _windowed_ex(lib, p, Opt(norm_weight=FAKE.value)) == INVALID          # a norm weight needs a gate
    assert _windowed_ex(lib, p, Opt(decay_floor=float("nan"))) == INVALID
    assert _windowed_ex(lib, p, Opt(alpha_mode=0), alpha=ctypes.c_void_p(0x10004)) == INVALID   # per channel: 16 B
    # with checkpoints a window holds a whole interval: a workspace that fits
    # 512 tokens of one sequence cannot take a window of 1,024
    st, row512 = _ws(lib, _params(seqlen=512))
    assert st == OK
    assert _windowed_ex(lib, p, Opt(checkpoints=ck.value, ckpt_every=1024, max_ckpts=4),
                        ws_bytes=row512) == WORKSPACE
    assert _windowed_ex(lib, p, Opt(gate=FAKE.value), ws_bytes=4096) == WORKSPACE


def test_calls_beyond_one_dispatch_are_unsupported(lib):
    """A grid of 2^32 work-items or more would wrap: such calls are refused before any launch."""
    huge = _params(seqlen=1 << 34, num_heads=1)     # 2^28 chunks x 256 threads
    assert lib.kda_chunk_fwd(ctypes.byref(huge), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE,
                             1 << 62, None) == UNSUPPORTED
    ok = _params(seqlen=1 << 20, num_heads=1)       # a plain large call passes this check (and fails later on
    assert lib.kda_chunk_fwd(ctypes.byref(ok), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None,
                             16, None) == WORKSPACE  # the 16-byte workspace, before any launch)
    assert lib.kda_decode_step(1 << 20, 32, 128, 128, 1.0, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               None) == UNSUPPORTED
