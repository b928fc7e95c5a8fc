"""Encoders that turn real values into the cache byte formats.

Formats (DeepSeek V4.1 Flash summary, page "DeepSeek V4.1 Flash 如何靠压缩 KV
缓存实现小模型干翻大模型", section on FP4 quantisation): main KV and the
indexer Q/K are FP4 E2M1 with one E4M3 scale per 16 channels and no second
level global scale; the sliding window stays 8 bit (E4M3 here).

Encoding is only how synthetic inputs are produced; the hot path never
encodes. The quantiser reading used here:

* block scale byte = E4M3 round-to-nearest-even of amax/6 (6 is the largest
  E2M1 magnitude), saturating at 448; amax == 0 gives scale byte 0;
* each value x is divided by the decoded scale and rounded to the nearest
  E2M1 magnitude with ties to the even mantissa, saturating at 6; the sign
  bit is x < 0 (so a negative value that rounds to zero gives code 0x8);
* two codes per byte, the even channel in the low nibble.

E4M3 rounding is delegated to torch's ``float8_e4m3fn`` conversion (a library
routine), which rounds to nearest even but maps out-of-range values to NaN,
hence the explicit clamp to +-448 first.
"""

from __future__ import annotations

import numpy as np
import torch

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def encode_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float values to OCP E4M3 ("fn") bytes, RNE, saturating at +-448."""
    x = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _e4m3_values_of(b: np.ndarray) -> np.ndarray:
    """float32 value of E4M3 bytes, via torch's float8 dtype (library decode)."""
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float32).numpy()


def _e2m1_magnitude_code(y: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude code (0..7) of |y|, ties to even mantissa, saturating.

    The E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7). Between
    two neighbours the midpoint goes to the code with even mantissa bit, i.e.
    the even code: 0.25->0, 0.75->2, 1.25->2, 1.75->4, 2.5->4, 3.5->6, 5->6.
    """
    a = np.abs(y)
    code = (
        (a > 0.25).astype(np.uint8)
        + (a >= 0.75)
        + (a > 1.25)
        + (a >= 1.75)
        + (a > 2.5)
        + (a >= 3.5)
        + (a > 5.0)
    )
    return code.astype(np.uint8)


def encode_fp4_blocks(x: np.ndarray):
    """Quantise ``x[..., C]`` (C a multiple of 16) to FP4 E2M1 + E4M3/16 scales.

    Returns ``(codes, scales)``: ``codes`` uint8 ``[..., C/2]`` with channel
    2j in the low nibble of byte j and 2j+1 in the high nibble; ``scales``
    uint8 ``[..., C/16]``, one E4M3 byte per 16 consecutive channels.
    """
    x = np.asarray(x, dtype=np.float32)
    C = x.shape[-1]
    if C % 16:
        raise ValueError("channel count must be a multiple of 16")
    lead = x.shape[:-1]
    blocks = x.reshape(*lead, C // 16, 16)
    amax = np.abs(blocks).max(axis=-1)
    scale_b = encode_e4m3(amax / np.float32(E2M1_MAX))
    scale_v = _e4m3_values_of(scale_b)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(scale_v[..., None] > 0, blocks / scale_v[..., None], np.float32(0))
    mag = _e2m1_magnitude_code(y)
    sign = (blocks < 0).astype(np.uint8) << 3
    nib = (mag | sign).reshape(*lead, C)
    codes = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return codes, scale_b.astype(np.uint8)
