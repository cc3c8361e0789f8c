"""Products of compressed weights with activations for any number of rows.

Up to FUSED_MAX_ROWS activation rows (the decode phase of inference) the
product is the fused decode + product (decode_gemm_tiles for tensors in tile
order, else decode_gemm): the bf16 weights are never written. With
more rows (prefill) the product, not the decode, dominates a layer's time, so
the layer is decoded once to bf16 and each projection is one library GEMM --
weights expanded right before the block that uses them [EntQuant,
"Float8@2bits ...", technical summary §2 "Decodificación en Tiempo de
Inferencia"].
"""
from __future__ import annotations

import numpy as np

from . import (EINVAL, KIND_BF16EXP, LAYOUT_TILES, OUT_BF16, EntqError, Plan, _gemm_io, decode,
               decode_gemm, decode_gemm_tiles)

FUSED_MAX_ROWS = 64


def linear(p: Plan, compressed, scales, xs, ys, weights=None, chunk_status=None, stream=None,
           workspace=None):
    """Y_t = X_t . W_t^T for every tensor t of the plan (xs[t]: device
    bfloat16 [m, >= cols]; ys[t]: device float32 [m, >= rows]; the same m for
    all). m <= FUSED_MAX_ROWS: decode_gemm_tiles when the plan's tensors are
    in tile order, else decode_gemm (workspace as there). More rows:
    the bf16 decode into `weights` (a device tensor of 2-byte elements, at
    least out_elems; allocated when None), then per tensor one library GEMM
    of the bf16 operands with fp32 accumulation and fp32 results, all on
    `stream` (a torch stream, a raw stream handle, or None for the current
    stream)."""
    import torch
    _gemm_io(p, xs, ys)  # shapes, dtypes and devices, as for the fused call
    m = xs[0].shape[0] if xs else 0
    tiles = bool(np.any(p.tensors["kind"] & LAYOUT_TILES))
    if m <= FUSED_MAX_ROWS:
        fused = decode_gemm_tiles if tiles else decode_gemm
        fused(p, compressed, scales, xs, ys, chunk_status, stream, workspace)
        return
    if p.adaptive:
        raise EntqError(EINVAL, "linear takes plans with per-tensor tables")
    if np.any((p.tensors["kind"] & 0xFF) == KIND_BF16EXP):
        raise EntqError(EINVAL, "linear takes Int8 and E4M3 tensors; exponent streams use "
                                "decode_gemm_bf16_split")
    own = weights is None
    if own:
        weights = torch.empty(p.out_elems, dtype=torch.int16, device=p.device)
    decode(p, compressed, weights, OUT_BF16, scales, chunk_status, stream)
    w = weights.view(torch.bfloat16)
    if stream is None:
        s = torch.cuda.current_stream(p.device)
    elif isinstance(stream, int):  # a raw stream handle, 0 for the null stream
        s = (torch.cuda.ExternalStream(stream, device=p.device) if stream
             else torch.cuda.default_stream(p.device))
    else:
        s = stream
    if own:
        weights.record_stream(s)  # allocated here, used on s
    with torch.cuda.stream(s):
        for t in range(p.n_tensors):
            rows, cols = int(p.tensors[t]["rows"]), int(p.tensors[t]["cols"])
            if rows * cols == 0:
                continue
            off = int(p.tensors[t]["out_elem_offset"])
            wt = w[off:off + rows * cols].view(rows, cols)
            ys[t][:, :rows].copy_(torch.mm(xs[t][:, :cols], wt.t(), out_dtype=torch.float32))
