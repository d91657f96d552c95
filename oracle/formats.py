"""Expert record layout and the decoders of the expert weight formats.

[PE] "What does Paged Experts actually do?": the feature supports bf16,
block-FP8 and GPTQ (int4) experts, and a Qwen3-30B-A3B expert is a SwiGLU FFN
of 3 x 2048 x 768 weights ([PE] "Why is it fast when experts keep crossing
PCIe?"). [PE] "Can paging change the model's outputs?": every per-expert
tensor (weights, scales, zero points) must be paged together, or a paged-in
expert silently runs with another expert's values. So each expert is ONE
contiguous record and one page-in moves all of it.

Record of one expert (H = hidden, I = intermediate), in this order:
  W13  = [W_gate; W_up]   2I rows x H columns, row-major (reduction dim H contiguous)
  W_d                      H rows x I columns, row-major (reduction dim I contiguous)
  then, per format, the scale and zero-point tables below.
The record stride is the payload rounded up to a multiple of 256 bytes; the
padding is zero.

Formats (readings where the pages name a format but not its layout):
  f32   : float32 weights.
  bf16  : bfloat16 weights.
  fp8   : OCP float8 e4m3fn codes (bias 7, max 448, no infinities, NaN = S.1111.111),
          weight-only; W = decode(q) * scale[r // 128][c // 128], float32 scales
          over 128x128 tiles of each matrix; scales of W13 [2I/128][H/128],
          then of W_d [H/128][I/128].
  int4  : asymmetric, groups of 128 along the reduction dim, w = (q - z) * s,
          q in 0..15, s and z float16; 8 codes per little-endian uint32 word
          along the reduction dim, the low nibble holding the lower index.
          Tables: scales W13 [2I][H/128], scales W_d [H][I/128], zeros W13
          [2I][H/128], zeros W_d [H][I/128].
  mxfp4 : OCP microscaling FP4: blocks of 32 consecutive weights along the
          reduction dim share one E8M0 scale byte (2^(byte - 127), 255 = NaN);
          each weight is an E2M1 code (sign 1 bit, exponent 2 bits with bias
          1, mantissa 1 bit; exponent 0 is subnormal: m/2); two codes per byte,
          the low nibble holding the lower index. Tables: scales W13
          [2I][H/32], scales W_d [H][I/32]. ([PE] "What does Paged Experts
          actually do?" lists MXFP4 among the formats of the follow-up work.)
"""
import numpy as np

F32, BF16, FP8, INT4, MXFP4 = 0, 1, 2, 3, 4
NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8_e4m3_b128", INT4: "int4_asym_g128", MXFP4: "mxfp4_e2m1_b32"}


def _sections(fmt, H, I):
    """(name, dtype, shape) of each section of a record, in order."""
    R13, C13, Rd, Cd = 2 * I, H, H, I
    if fmt == F32:
        return [("w13", np.float32, (R13, C13)), ("wd", np.float32, (Rd, Cd))]
    if fmt == BF16:
        return [("w13", np.uint16, (R13, C13)), ("wd", np.uint16, (Rd, Cd))]
    if fmt == FP8:
        return [("w13", np.uint8, (R13, C13)), ("wd", np.uint8, (Rd, Cd)),
                ("s13", np.float32, (R13 // 128, C13 // 128)),
                ("sd", np.float32, (Rd // 128, Cd // 128))]
    if fmt == INT4:
        return [("w13", np.uint32, (R13, C13 // 8)), ("wd", np.uint32, (Rd, Cd // 8)),
                ("s13", np.float16, (R13, C13 // 128)), ("sd", np.float16, (Rd, Cd // 128)),
                ("z13", np.float16, (R13, C13 // 128)), ("zd", np.float16, (Rd, Cd // 128))]
    if fmt == MXFP4:
        return [("w13", np.uint8, (R13, C13 // 2)), ("wd", np.uint8, (Rd, Cd // 2)),
                ("s13", np.uint8, (R13, C13 // 32)), ("sd", np.uint8, (Rd, Cd // 32))]
    raise ValueError("unknown format %r" % (fmt,))


def payload_bytes(fmt, H, I):
    return sum(np.dtype(dt).itemsize * int(np.prod(sh)) for _, dt, sh in _sections(fmt, H, I))


def record_stride(fmt, H, I):
    p = payload_bytes(fmt, H, I)
    return (p + 255) // 256 * 256


def split_record(rec, fmt, H, I):
    """Views of the sections of one record (uint8 array of at least payload bytes)."""
    rec = np.asarray(rec, dtype=np.uint8)
    out, off = {}, 0
    for name, dt, sh in _sections(fmt, H, I):
        n = np.dtype(dt).itemsize * int(np.prod(sh))
        out[name] = rec[off:off + n].view(dt).reshape(sh)
        off += n
    return out


# ---------------------------------------------------------------- decoders

def bf16_to_f64(u16):
    """bfloat16 bit patterns -> float64 (exact: bf16 is the top half of a float32)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def fp8_e4m3fn_to_f64(codes):
    """OCP e4m3fn codes -> float64, from the definition of the encoding.

    sign 1 bit, exponent 4 bits (bias 7), mantissa 3 bits. Exponent 0 is
    subnormal: m/8 * 2^-6. Exponent 1..15 is (1 + m/8) * 2^(e-7), except
    exponent 15 with mantissa 7, which is NaN (there are no infinities).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, v)


def f16_to_f64(h):
    return np.asarray(h, dtype=np.float16).astype(np.float64)


def int4_unpack(words):
    """uint32 words [R][C/8] -> codes int64 [R][C]; nibble n of word w is code 8w+n."""
    w = np.asarray(words, dtype=np.uint32).astype(np.int64)
    R, W = w.shape
    shifts = 4 * np.arange(8)
    return ((w[:, :, None] >> shifts[None, None, :]) & 0xF).reshape(R, W * 8)


def e2m1_to_f64(codes):
    """OCP E2M1 codes (0..15) -> float64, from the definition of the encoding:
    sign 1 bit, exponent 2 bits (bias 1), mantissa 1 bit; exponent 0 is
    subnormal, m/2; exponent 1..3 is (1 + m/2) * 2^(e-1). No infinities or NaN."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m / 2.0, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def e8m0_to_f64(b):
    """OCP E8M0 scale bytes -> float64: 2^(b - 127); 255 is NaN."""
    b = np.asarray(b).astype(np.int64)
    return np.where(b == 255, np.nan, np.exp2(b - 127.0))


def nibbles_unpack(b):
    """uint8 [R][C/2] -> codes int64 [R][C]; byte j holds codes 2j (low nibble) and 2j+1."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    R, B = b.shape
    out = np.empty((R, 2 * B), dtype=np.int64)
    out[:, 0::2] = b & 0xF
    out[:, 1::2] = b >> 4
    return out


def _dequant_mxfp4(codes, scales):
    v = e2m1_to_f64(nibbles_unpack(codes))
    return v * np.repeat(e8m0_to_f64(scales), 32, axis=1)


def _dequant_fp8(q, scales):
    R, C = q.shape
    v = fp8_e4m3fn_to_f64(q)
    s = scales.astype(np.float64)
    return v * np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:R, :C]


def _dequant_int4(words, scales, zeros):
    q = int4_unpack(words).astype(np.float64)
    s = np.repeat(f16_to_f64(scales), 128, axis=1)
    z = np.repeat(f16_to_f64(zeros), 128, axis=1)
    return (q - z) * s


def decode_record(rec, fmt, H, I):
    """One expert record -> (W_gate [I,H], W_up [I,H], W_down [H,I]) in float64."""
    sec = split_record(rec, fmt, H, I)
    if fmt == F32:
        w13, wd = sec["w13"].astype(np.float64), sec["wd"].astype(np.float64)
    elif fmt == BF16:
        w13, wd = bf16_to_f64(sec["w13"]), bf16_to_f64(sec["wd"])
    elif fmt == FP8:
        w13, wd = _dequant_fp8(sec["w13"], sec["s13"]), _dequant_fp8(sec["wd"], sec["sd"])
    elif fmt == INT4:
        w13 = _dequant_int4(sec["w13"], sec["s13"], sec["z13"])
        wd = _dequant_int4(sec["wd"], sec["sd"], sec["zd"])
    elif fmt == MXFP4:
        w13, wd = _dequant_mxfp4(sec["w13"], sec["s13"]), _dequant_mxfp4(sec["wd"], sec["sd"])
    else:
        raise ValueError(fmt)
    return w13[:I], w13[I:], wd
