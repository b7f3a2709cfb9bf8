"""The converter facts the attention kernels rely on, checked on the device at hand
through nvfp4_hw_self_check: gfx950's FP32 -> FP8 (E4M3) convert rounds every
binary32 in [0, 448] to nearest even exactly as the UE4M3 rounding of the block
scales does (the P block-pattern estimate uses it), and its FP8 -> FP32 convert
gives every scale byte below 127 its UE4M3 value (the block-scale decode uses it)."""
import pytest

pytestmark = pytest.mark.gpu


def test_converters_match_ue4m3(gpu):
    rounding, decode = gpu.hw_self_check()
    assert rounding == 0, f"{rounding} binary32 values in [0, 448] round differently"
    assert decode == 0, f"{decode} scale bytes decode differently"
