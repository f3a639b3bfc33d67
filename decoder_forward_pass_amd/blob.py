"""Pack a model's weights into the library's blob format (host-side marshalling).

The library defines the blob layout (``dec_weight_entry``): each entry's byte
offset, dtype and shape. This module copies arrays into those places. 4-bit
values are packed two per byte, column 2b in the low nibble and column 2b+1 in
the high nibble ("Candle model runner" section 2.5 "Int4 weights"); signed
values as 4-bit two's complement ("Candle model runner" 2.5).
"""

from __future__ import annotations

import numpy as np


def pack_uint4(q) -> np.ndarray:
    """[out, in] codes 0..15 (one per element) -> [out, in/2] bytes."""
    q = np.asarray(q, dtype=np.uint8)
    if q.shape[-1] % 2:
        raise ValueError("the input dimension must be even")
    if q.max(initial=0) > 15:
        raise ValueError("codes must be 0..15")
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def pack_int4_sym(q) -> np.ndarray:
    """[out, in] signed values -8..7 (one per element) -> [out, in/2] bytes of 4-bit two's complement."""
    q = np.asarray(q)
    if q.shape[-1] % 2:
        raise ValueError("the input dimension must be even")
    if q.size and (q.min() < -8 or q.max() > 7):
        raise ValueError("values must be -8..7")
    n = (q.astype(np.int16) & 15).astype(np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def _source(weights, name: str, layer: int):
    if name == "embed":
        return weights.embed
    if name == "final_norm":
        return weights.final_norm
    return weights.layers[layer][name]


def pack_blob(cfg, weights) -> np.ndarray:
    """The blob bytes (uint8) for ``weights`` (a synthetic.Weights) under ``cfg``."""
    from .binding import (DEC_F32, DEC_INT4_SYM_G32, DEC_UINT4_G32, dec_weight_bytes, dec_weight_count,
                          dec_weight_entry)

    buf = np.zeros(dec_weight_bytes(cfg), dtype=np.uint8)
    for i in range(dec_weight_count(cfg)):
        e = dec_weight_entry(cfg, i)
        src = _source(weights, e.name.decode(), e.layer)
        if e.dtype == DEC_UINT4_G32:
            codes = pack_uint4(src.q).reshape(-1)
            buf[e.offset:e.offset + e.bytes] = codes
            buf[e.scale_offset:e.scale_offset + e.group_bytes] = np.ascontiguousarray(src.scale, np.uint16).view(np.uint8).reshape(-1)
            buf[e.zp_offset:e.zp_offset + e.group_bytes] = np.ascontiguousarray(src.zp, np.uint16).view(np.uint8).reshape(-1)
            continue
        if e.dtype == DEC_INT4_SYM_G32:
            buf[e.offset:e.offset + e.bytes] = pack_int4_sym(src.q).reshape(-1)
            buf[e.scale_offset:e.scale_offset + e.group_bytes] = np.ascontiguousarray(src.scale, np.uint16).view(np.uint8).reshape(-1)
            continue
        want = np.float32 if e.dtype == DEC_F32 else np.uint16
        arr = np.ascontiguousarray(src, dtype=want)
        if arr.size != e.rows * e.cols:
            raise ValueError(f"entry {e.name.decode()} (layer {e.layer}): {arr.size} values, expected {e.rows * e.cols}")
        buf[e.offset:e.offset + e.bytes] = arr.view(np.uint8).reshape(-1)
    return buf
