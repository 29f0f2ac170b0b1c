"""Bit-exact tests of the device decoders the GEMM kernels use, over every code."""
import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsg
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def test_decode_e4m3_every_code():
    codes = torch.arange(256, dtype=torch.uint8, device="cuda")
    out = torch.empty(256, dtype=torch.float32, device="cuda")
    bsg.decode_e4m3(codes, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = O.decode_e4m3(np.arange(256))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].astype(np.float32).view(np.uint32))


def test_decode_nvfp4_every_byte_and_scale():
    # every packed byte (two E2M1 codes) against every finite E4M3 scale code: for each scale, one
    # 512-element row holding bytes 0..255 (32 blocks of 16 sharing that scale)
    scodes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    packed = np.tile(np.arange(256, dtype=np.uint8), len(scodes))
    scales = np.repeat(scodes, 32)
    n = 2 * packed.size
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    bsg.decode_nvfp4(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(), out, n)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    vals = O.dequant_nvfp4(packed[None, :], scales[None, :], n)[0]
    want = O.round_to_bf16_bits(vals)
    # exact products: the oracle's rounding is the identity here, so bits must agree everywhere
    assert np.array_equal(got, want), f"{int((got != want).sum())} mismatching products"


@pytest.mark.gpu
def test_decode_nvfp4_f16_every_byte_and_scale():
    # the tiled kernels' fp16 route: every packed byte against every E4M3 scale code (NaN codes too),
    # one 512-element row per scale code; the result is e2m1 * e4m3 * 2^-7, exact in fp16
    scodes = np.arange(256, dtype=np.uint8)
    packed = np.tile(np.arange(256, dtype=np.uint8), len(scodes))
    scales = np.repeat(scodes, 32)
    n = 2 * packed.size
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    bsg.decode_nvfp4_f16(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(), out, n)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    vals = O.dequant_nvfp4(packed[None, :], scales[None, :], n)[0] * 2.0 ** -7
    nan = np.isnan(vals)
    assert nan.sum() == 2 * 512
    got_nan = ((got & 0x7C00) == 0x7C00) & ((got & 0x03FF) != 0)
    assert np.array_equal(got_nan, nan)
    want = O.round_to_f16_bits(np.where(nan, 0.0, vals))
    # every finite product is exact in fp16 (subnormals included): bits agree, signed zeros too
    assert np.array_equal(got[~nan], want[~nan]), f"{int((got[~nan] != want[~nan]).sum())} mismatching"
    assert np.array_equal(O.bits_to_f64(want[~nan], "f16"), vals[~nan])


@pytest.mark.gpu
def test_decode_nvfp4_f16_rejects_bad_sizes():
    z = torch.zeros(64, dtype=torch.uint8, device="cuda")
    o = torch.zeros(128, dtype=torch.int16, device="cuda")
    with pytest.raises(bsg.BsgError) as e:
        bsg.decode_nvfp4_f16(z, z, o, 48)
    assert e.value.status_name == "BSG_ERR_SHAPE"
