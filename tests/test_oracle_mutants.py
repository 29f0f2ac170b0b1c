"""Plant plausible mistakes in the oracle (on the CPU) and check that some pin catches each one."""
import numpy as np
import pytest

from oracle import oracle as O
from oracle_pins import ALL_PINS

_orig = {name: getattr(O, name) for name in ("decode_e4m3", "decode_e8m0", "decode_e2m1", "unpack_e2m1",
                                             "dequant_mxfp8", "dequant_nvfp4", "contract", "epilogue",
                                             "round_to_bf16_bits")}


def _e4m3_bias_off(codes):
    return _orig["decode_e4m3"](codes) * 0.5


def _e4m3_subnormal_as_normal(codes):
    c = np.asarray(codes).astype(np.int64)
    v = _orig["decode_e4m3"](codes)
    e, m, s = (c >> 3) & 0xF, c & 7, (c >> 7) & 1
    wrong = np.ldexp(1.0 + m / 8.0, -7) * np.where(s == 1, -1, 1)
    return np.where((e == 0) & (m != 0), wrong, v)


def _e8m0_bias_off(codes):
    return _orig["decode_e8m0"](codes) * 2.0


def _e2m1_mantissa_weight(codes):
    c = np.asarray(codes).astype(np.int64)
    e, m, s = (c >> 1) & 3, c & 1, (c >> 3) & 1
    mag = np.where(e == 0, m / 2.0, np.ldexp(1.0 + m / 4.0, e - 1))
    return np.where(s == 1, -mag, mag)


def _nibbles_swapped(packed, K):
    out = _orig["unpack_e2m1"](packed, K)
    return np.ascontiguousarray(out.reshape(out.shape[0], -1, 2)[:, :, ::-1].reshape(out.shape))


def _mx_block_index_tiled(codes, scales):
    R, K = codes.shape
    return O.decode_e4m3(codes) * np.tile(O.decode_e8m0(scales), (1, 32))


def _mx_block_off_by_one(codes, scales):
    s = np.roll(O.decode_e8m0(scales), 1, axis=1)
    return O.decode_e4m3(codes) * np.repeat(s, 32, axis=1)


def _nv_block_size_32(packed, scales, K):
    s = O.decode_e4m3(scales)[:, : K // 32]
    return O.decode_e2m1(O.unpack_e2m1(packed, K)) * np.repeat(s, 32, axis=1)


def _contract_transposed(a, b):
    acc, S = _orig["contract"](a, b)
    return (acc.T if acc.shape[0] == acc.shape[1] else acc[::-1]), S


def _contract_drops_last_k(a, b):
    return _orig["contract"](a[:, :-1], b[:, :-1])


def _epi_no_bias(acc, alpha, bias, silu):
    return _orig["epilogue"](acc, alpha, None, silu)


def _epi_alpha_after_silu(acc, alpha, bias, silu):
    y = _orig["epilogue"](acc, np.float32(1.0), bias, silu)
    return float(np.float32(alpha)) * y


def _epi_silu_sign(acc, alpha, bias, silu):
    y = _orig["epilogue"](acc, alpha, bias, False)
    return y / (1.0 + np.exp(y)) if silu else y


def _epi_alpha_f64(acc, alpha, bias, silu):
    y = acc * 0.1000000000000001 / 0.1 * float(np.float32(alpha))
    return _orig["epilogue"](y, np.float32(1.0), bias, silu)


def _bf16_truncate(y):
    f32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def _bf16_via_f32(y):
    import torch
    return torch.from_numpy(np.asarray(y, np.float64).astype(np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


MUTANTS = {
    "e4m3_bias_off_by_one": ("decode_e4m3", _e4m3_bias_off),
    "e4m3_subnormals_as_normals": ("decode_e4m3", _e4m3_subnormal_as_normal),
    "e8m0_bias_off_by_one": ("decode_e8m0", _e8m0_bias_off),
    "e2m1_wrong_mantissa_weight": ("decode_e2m1", _e2m1_mantissa_weight),
    "e2m1_nibbles_swapped": ("unpack_e2m1", _nibbles_swapped),
    "mx_scale_index_k_mod_blocks": ("dequant_mxfp8", _mx_block_index_tiled),
    "mx_scale_block_shifted": ("dequant_mxfp8", _mx_block_off_by_one),
    "nv_block_size_32": ("dequant_nvfp4", _nv_block_size_32),
    "contract_transposed": ("contract", _contract_transposed),
    "contract_drops_a_term": ("contract", _contract_drops_last_k),
    "epilogue_drops_bias": ("epilogue", _epi_no_bias),
    "epilogue_alpha_after_silu": ("epilogue", _epi_alpha_after_silu),
    "epilogue_silu_sign": ("epilogue", _epi_silu_sign),
    "epilogue_alpha_perturbed": ("epilogue", _epi_alpha_f64),
    "bf16_truncation": ("round_to_bf16_bits", _bf16_truncate),
    "bf16_double_rounding_via_f32": ("round_to_bf16_bits", _bf16_via_f32),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
