"""Pins for the oracle's byte decoders (O0): every code, against torch's own
dtype conversions (library routine, exhaustive)."""
import numpy as np
import torch


def test_fp8_e4m3fn_all_codes(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.decode_fp8(codes.numpy())
    nan_ref = np.isnan(ref)
    assert nan_ref.sum() == 2 and set(np.nonzero(nan_ref)[0]) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(got), nan_ref)
    assert np.array_equal(got[~nan_ref], ref[~nan_ref])
    # the integers the workloads draw are exact
    for v in range(-8, 9):
        b = torch.tensor([float(v)]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert orc.decode_fp8(b)[0] == v


def test_bf16_all_codes(orc):
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.decode_bf16(codes.numpy().view(np.uint16))
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref)
    assert np.array_equal(got[~nan_ref], ref[~nan_ref])
