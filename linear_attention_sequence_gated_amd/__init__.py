"""KDA (Kimi Delta Attention) token mixer on MI355X: Python binding of libkda.so.

The hot path -- chunked prefill (``chunk_fwd``) and the single-token decode
step (``decode_step``) -- runs entirely in hand-written HIP kernels for gfx950
behind the C ABI of include/kda.h; this package only marshals arguments.
"""
from ._lib import (EXPORTED, KDA_DTYPE_BF16, KDA_DTYPE_F32, KDA_ERR_INVALID_ARG, KDA_ERR_RANGE, ChunkOptions, ChunkParams, ChunkPlan, DecodeOptions, KdaError, Prefill, chunk_fwd, chunk_fwd_noalloc,
                   chunk_fwd_windowed,
                   chunk_plan, decode_step, library_path, load, status_string, workspace_size)

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_windowed", "chunk_plan", "decode_step", "Prefill", "workspace_size", "status_string", "load",
           "library_path", "KdaError", "ChunkParams", "ChunkOptions", "ChunkPlan", "DecodeOptions", "EXPORTED", "KDA_DTYPE_F32", "KDA_DTYPE_BF16", "KDA_ERR_RANGE", "KDA_ERR_INVALID_ARG"]
