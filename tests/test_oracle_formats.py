"""Oracle decoders pinned to library conversions and hand-packed words, plus the
generator <-> oracle record layout round trip."""
import numpy as np
import pytest
import torch

from oracle import formats
from workloads import gen


def test_fp8_all_256_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.fp8_e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                              # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_bf16_vs_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 65536, size=20000, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # finite only
    ours = formats.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_int4_hand_packed_words():
    w = np.array([[0x76543210, 0xFEDCBA98]], dtype=np.uint32)
    assert formats.int4_unpack(w).tolist() == [list(range(16))]
    w = np.array([[0x0000000F]], dtype=np.uint32)
    assert formats.int4_unpack(w).tolist() == [[15, 0, 0, 0, 0, 0, 0, 0]]
    # dequant of one group of 128: codes 0..15 repeating, s = 0.5, z = 3.25
    q = np.tile(np.arange(16), 8)
    words = np.zeros((1, 16), dtype=np.uint32)
    for i, c in enumerate(q):
        words[0, i // 8] |= np.uint32(c) << np.uint32(4 * (i % 8))
    deq = formats._dequant_int4(words, np.array([[0.5]], np.float16), np.array([[3.25]], np.float16))
    assert np.array_equal(deq[0], (q - 3.25) * 0.5)


def test_fp8_tile_scales_hand_built():
    # one 128x128 tile of code 0x38 (= 1.0) with scale 0.25, a second with scale 2
    q = np.full((128, 256), 0x38, dtype=np.uint8)
    s = np.array([[0.25, 2.0]], dtype=np.float32)
    d = formats._dequant_fp8(q, s)
    assert np.all(d[:, :128] == 0.25) and np.all(d[:, 128:] == 2.0)


QWEN = (2048, 768)


def test_record_sizes_qwen_shape():
    H, I = QWEN
    assert formats.payload_bytes(formats.BF16, H, I) == 9437184
    assert formats.payload_bytes(formats.FP8, H, I) == 4718592 + 1152
    assert formats.payload_bytes(formats.INT4, H, I) == 2359296 + 73728 + 73728
    # [PE] 'Why is it fast ...': an FP8 expert is about 4.72 MB with scales ignored
    assert abs(3 * H * I / 1e6 - 4.72) < 0.005
    # the page's 2.43 MB int4 expert is int4 codes + one fp16 scale per 128 (symmetric)
    assert 3 * H * I // 2 + 2 * 3 * H * I // 128 == 2433024
    for f in (formats.F32, formats.BF16, formats.FP8, formats.INT4):
        assert formats.record_stride(f, H, I) == gen.record_stride(f, H, I)
        assert formats.record_stride(f, H, I) % 256 == 0


@pytest.mark.parametrize("fmt,tol", [(formats.F32, 0.0), (formats.BF16, 2.0 ** -8),
                                     (formats.FP8, None), (formats.INT4, None)])
def test_generator_roundtrip(fmt, tol):
    """Records the generator packs decode (oracle) to the values it packed,
    within the format's own quantisation error: this pins the layout the two
    independent implementations agree on."""
    H, I = 256, 384
    rng = np.random.default_rng(11)
    w13 = (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32)
    wd = (rng.standard_normal((H, I)) * 0.02).astype(np.float32)
    w13[:3, :5] = 0.0
    rec = gen.encode_record(fmt, w13, wd)
    g, u, d = formats.decode_record(rec, fmt, H, I)
    for got, ref in ((g, w13[:I]), (u, w13[I:]), (d, wd)):
        ref = ref.astype(np.float64)
        err = np.abs(got - ref)
        if fmt == formats.F32:
            assert np.array_equal(got, ref)
        elif fmt == formats.BF16:
            assert np.all(err <= np.abs(ref) * tol)
        elif fmt == formats.FP8:
            R, C = ref.shape
            amax = np.abs(ref.reshape(R // 128, 128, C // 128, 128)).max(axis=(1, 3))
            s = np.repeat(np.repeat(amax / 448.0, 128, 0), 128, 1)
            # e4m3 has 3 mantissa bits: half an ulp is 2^-4 relative, 2^-10 * s absolute at the bottom
            assert np.all(err <= np.maximum(np.abs(ref) * 2.0 ** -4, s * 2.0 ** -10) * 1.0001)
        else:
            R, C = ref.shape
            grp = ref.reshape(R, C // 128, 128)
            s = (grp.max(2) - grp.min(2)) / 15.0
            bound = np.repeat(s, 128, axis=1) * 0.5 * 1.02 + 1e-4 * np.abs(ref).max()
            assert np.all(err <= bound)
    # padding is zero
    assert not rec[formats.payload_bytes(fmt, H, I):].any()


def test_e2m1_value_table():
    """The sixteen E2M1 values of the OCP microscaling FP4 element type, listed
    (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; code 8 is negative zero)."""
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
             -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    got = formats.e2m1_to_f64(np.arange(16))
    assert np.array_equal(got, np.array(table))
    assert np.signbit(got[8])


def test_e8m0_scale_bytes():
    got = formats.e8m0_to_f64(np.array([0, 1, 126, 127, 128, 254, 255]))
    assert np.array_equal(got[:6], [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127])
    assert np.isnan(got[6])


def test_e8m0_all_bytes_vs_torch():
    """Every E8M0 byte against torch's float8_e8m0fnu conversion (a library
    routine written from the same OCP definition)."""
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).float().double().numpy()
    got = formats.e8m0_to_f64(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[:255], ref[:255])


def test_mxfp4_hand_built_record():
    """A record written byte by byte: nibble order, block scales and sections."""
    H, I = 64, 32                       # W13 [64][64], W_d [64][32]
    rec = np.zeros(formats.record_stride(formats.MXFP4, H, I), np.uint8)
    sec = formats.split_record(rec, formats.MXFP4, H, I)
    sec["w13"][0, 0] = 0x21             # codes 1 (low nibble) and 2 -> 0.5, 1.0
    sec["w13"][0, 16] = 0xF7            # element 32: code 7 (6.0), element 33: code 15 (-6.0)
    sec["s13"][0, 0] = 128              # block 0 of row 0 scaled by 2
    sec["s13"][0, 1] = 125              # block 1 scaled by 1/4
    sec["s13"][1:, :] = 127
    sec["wd"][5, 3] = 0x9A              # W_d row 5, elements 6 and 7: code 10 (-1.0), code 9 (-0.5)
    sec["sd"][:, :] = 127
    sec["sd"][5, 0] = 129               # x4
    g, u, d = formats.decode_record(rec, formats.MXFP4, H, I)
    assert g[0, 0] == 1.0 and g[0, 1] == 2.0 and g[0, 2] == 0.0
    assert g[0, 32] == 1.5 and g[0, 33] == -1.5
    assert d[5, 6] == -4.0 and d[5, 7] == -2.0 and d[5, 8] == 0.0
    assert np.count_nonzero(g) == 4 and np.count_nonzero(u) == 0 and np.count_nonzero(d) == 2
    # payload: 3HI/2 code bytes + one scale byte per 32 weights
    assert formats.payload_bytes(formats.MXFP4, 2048, 768) == 2359296 + 147456


def test_mxfp4_generator_roundtrip():
    """Records the generator packs decode to the packed values within two units
    of the block scale: the shared exponent floor(log2(amax)) - 2 puts the block
    maximum in [4, 8) units, so values above 6 units saturate at 6 (error < 2),
    and below that the widest step (4 -> 6) rounds with error <= 1."""
    H, I = 256, 384
    rng = np.random.default_rng(12)
    w13 = (rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32)
    wd = (rng.standard_normal((H, I)) * 0.02).astype(np.float32)
    w13[:2, :40] = 0.0
    rec = gen.encode_record(formats.MXFP4, w13, wd)
    assert rec.size == gen.record_stride(formats.MXFP4, H, I) == formats.record_stride(formats.MXFP4, H, I)
    g, u, d = formats.decode_record(rec, formats.MXFP4, H, I)
    for got, ref in ((g, w13[:I]), (u, w13[I:]), (d, wd)):
        ref = ref.astype(np.float64)
        R, C = ref.shape
        amax = np.abs(ref.reshape(R, C // 32, 32)).max(axis=2)
        scale = np.exp2(np.floor(np.log2(np.maximum(amax, 1e-38))) - 2)
        unit = np.repeat(np.where(amax > 0, scale, 0.0), 32, axis=1)
        small = np.abs(ref) <= 6 * unit
        assert np.all(np.abs(got - ref)[small] <= unit[small] * 1.0 + 1e-12)
        bound = unit * 2.0 + 1e-12
        assert np.all(np.abs(got - ref) <= bound)
        assert np.all(got[ref == 0] == 0)
