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
