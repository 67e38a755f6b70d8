"""Pins against numbers the pages print (tests/golden/pages_numbers.txt).

The roofline helpers must reproduce the page's H100 figures from its own
formula AI(decode, B) ~= 2B / bytes_per_weight; the effective-bit count comes
from "Low-precision LLM inference kernels" section 5; the E4M3 field widths of
its section 7 table fix the oracle's FP8 decoder (bias 2^(e-1)-1 = 7, three
mantissa bits: 1.0 is 0 0111 000, the smallest subnormal 2^-9).
"""
import os

from bit_gemm_w4_amd import roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.txt")


def _numbers():
    out = {}
    for line in open(GOLDEN):
        line = line.split("|")[0].strip()
        if not line or line.startswith("#"):
            continue
        name, *vals = line.split()
        out[name] = [float(v) for v in vals]
    return out


def test_critical_batch_and_ai():
    g = _numbers()
    ridge = g["h100_ridge_flop_per_byte"][0]
    assert round(roofline.critical_batch(ridge, 0.5)) == g["w4a16_critical_batch_h100"][0]
    assert roofline.ai_decode(1, 2.0) == g["ai_decode_bf16_bs1"][0]
    # the batch where AI reaches the ridge, by the formula, for INT4
    b = roofline.critical_batch(ridge, 0.5)
    assert abs(roofline.ai_decode(b, 0.5) - ridge) < 1e-9


def test_effective_bits():
    g = _numbers()
    assert roofline.effective_bits(4, 16, 128) == g["effective_bits_int4_g128_fp16"][0]


def test_ridge_of_spec_peaks():
    # MI355X dense BF16 2.5 PFLOP/s over 8 TB/s: 312.5 FLOP/byte; INT8/FP8 twice that
    assert roofline.ridge(roofline.PEAK_TFLOPS["bf16"], roofline.HBM_GBPS) == 312.5
    assert roofline.ridge(roofline.PEAK_TFLOPS["fp8"], roofline.HBM_GBPS) == 625.0


def test_e4m3_fields_fix_the_decoder(orc):
    s, e, m = (int(v) for v in _numbers()["e4m3_sign_exp_mantissa_bits"])
    assert s + e + m == 8
    bias = 2 ** (e - 1) - 1
    one = bias << m                                       # exponent field = bias, mantissa 0
    assert orc.e4m3_decode(one) == 1.0
    assert orc.e4m3_decode(1) == 2.0 ** (1 - bias - m)    # smallest subnormal
    assert orc.e4m3_decode(0x80 | one) == -1.0
    # largest finite: all-ones exponent with mantissa 110 (111 is NaN in the FN variant)
    assert orc.e4m3_decode((2 ** e - 1) << m | 0b110) == 2.0 ** (2 ** e - 1 - bias) * 1.75
