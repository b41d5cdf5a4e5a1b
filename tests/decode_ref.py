"""Decoding of block-scaled codes written from the format definitions alone,
for pinning the oracle: E2M1 from its bit fields, E4M3 through torch's
float8_e4m3fn view-cast, E8M0 as 2^(b - 127).  Shares nothing with the
oracle or the GPU library."""
import numpy as np
import torch

MXFP4, MXFP8, NVFP4 = 0, 1, 2
BLOCK = {MXFP4: 32, MXFP8: 32, NVFP4: 16}


def e2m1_value(c):
    """E2M1 from its fields: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    c = np.asarray(c, np.int64)
    e, m = (c >> 1) & 3, c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return np.where(c & 8, -mag, mag)


def e4m3_value(b):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(b, np.uint8)))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e8m0_value(b):
    b = np.asarray(b, np.int64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def numpy_dequantize(codes, scales, fmt, K, tsf=1.0):
    bs = BLOCK[fmt]
    if fmt == MXFP8:
        v = e4m3_value(codes[:, :K])
    else:
        lo, hi = codes & 0xF, codes >> 4
        v = np.empty((codes.shape[0], K))
        v[:, 0::2] = e2m1_value(lo[:, :K // 2])
        v[:, 1::2] = e2m1_value(hi[:, :K // 2])
    sc = scales[:, :K // bs]
    if fmt == NVFP4:
        s = e4m3_value(sc) * float(np.float32(tsf))
    else:
        s = e8m0_value(sc)
    return v * np.repeat(s, bs, axis=1)


def same_f64(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and \
        np.array_equal(np.nan_to_num(a, nan=0.0).view(np.uint64), np.nan_to_num(b, nan=0.0).view(np.uint64))
