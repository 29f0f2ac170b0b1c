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
