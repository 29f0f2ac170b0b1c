"""Bit-exact test of the device NVFP4 dequantisation the GEMM kernels use, over every code."""
import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsg
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.gpu
def test_decode_nvfp4_f16_every_byte_and_scale():
    # the GEMM kernels' dequantisation: every packed byte against every E4M3 scale code (NaN codes
    # too), one 512-element row per scale code; the result is e2m1 * e4m3 * 2^-8, exact in fp16
    scodes = np.arange(256, dtype=np.uint8)
    packed = np.tile(np.arange(256, dtype=np.uint8), len(scodes))
    scales = np.repeat(scodes, 32)
    n = 2 * packed.size
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    bsg.decode_nvfp4_f16(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(), out, n)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    vals = O.dequant_nvfp4(packed[None, :], scales[None, :], n)[0] * 2.0 ** -8
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
