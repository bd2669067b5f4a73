"""The division-free rounding rule of the quantizer's codes, checked on the CPU.

The kernels take the code of an fp16 value a in a group with fp16 scale s as
k = rint(fma(a, rcp(s), 768)) - 768 and claim k = rne(a / s) (round half to
even) wherever |a / s| < 16, beyond which every code saturates.  The group
quantization of "AI-Research-SKILLs AWQ 高级使用指南" (section
分组大小与零点量化) rounds the quotient to the nearest integer; ties decide
about 1 in 250 codes of fp16 weights, so the rule must reproduce them exactly.

This test emulates the arithmetic exactly in fp64 — a * rs is exact (11 x 24
significant bits), and fp32's grid on [512, 1024) is 2^-14 — for every finite
fp16 a against a spread of scales (normal and subnormal, with rcp taken as the
correctly rounded reciprocal and either fp32 neighbour, as the hardware
reciprocal is within one ulp).
"""
import numpy as np

_A = None


def _all_fp16():
    global _A
    if _A is None:
        pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
        _A = np.concatenate([pos, -pos[1:]])
    return _A


def _check_scale(s):
    a = _all_fp16()
    r0 = np.float32(1.0 / s)
    for rs32 in (r0, np.nextafter(r0, np.float32(0)), np.nextafter(r0, np.float32(np.inf))):
        t = a * float(rs32)                        # exact
        q = a / s
        inb = np.abs(t) < 240                       # 768 + t stays in [512, 1024)
        v = np.rint(t[inb] * 16384.0) / 16384.0     # fl32(768 + t) - 768
        k = np.rint(v)                              # rint(768 + .) - 768: 768 is even
        assert np.array_equal(k, np.rint(q[inb])), s
        # outside, the sum is beyond 768 +- 16 on the quotient's side: saturated codes
        assert np.all(np.sign(t[~inb]) == np.sign(q[~inb]))


def test_biased_quotient_matches_rne_on_all_fp16_weights():
    bits = list(range(1, 0x20, 3)) + list(range(0x0400, 0x7C00, 97)) + [0x3C00, 0x2E66, 0x1400, 0x7BFF]
    for b in bits:
        _check_scale(float(np.uint16(b).view(np.float16)))


def test_half_integer_quotients_are_present():
    # the rule is only interesting because exact ties occur: with a scale of few
    # significant bits every half-integer quotient below 16 is an fp16 weight
    a = _all_fp16()
    s = 0.1875
    q = a / s
    ties = np.abs(q) < 16
    assert np.count_nonzero((q[ties] - np.floor(q[ties])) == 0.5) == 32
