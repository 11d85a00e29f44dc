"""The quantizer kernels' step arithmetic equals the correctly rounded
definition (CPU only).

The page quantizer forms a step s16 = f16(f32(r / L)) with r = max - min and
L = 2^b - 1 levels (the asymmetric min/max group quantization of "Kitty --
Dynamic Channel-wise Mixed-Precision Keys", How it works / Prefill phase,
step 3, in the oracle's float32 reading), and the float32 reciprocal 1 / s
of that step.  The kernels use no division instruction:

* r / L as q0 = RN(r * RN(1 / L)), rem = RN(r - q0 L) (an FMA), and
  q = RN(q0 + rem * RN(1 / L)) (an FMA);
* 1 / s as y0 = v_rcp_f32(s) (within 1 ulp), then y = RN(y0 + RN(1 - s y0) y0)
  (two FMAs).

The running ranking mode's key statistics kernel sums a = k 2^24 and a^2
exactly in float64 (a split of a into two halves keeps every term and every
partial sum an exact float64, each a multiple of its own power of two); the
last test checks that against Python integers.

The first tests check both steps against exact rational arithmetic for
every input the kernels can meet.  Every operation scales exactly by powers of two while its
result stays a normal float32 (r <= 131008, 1 / s <= 2^24 for fp16 steps), so
all float32 significands of one binade cover r, and all fp16 significands (the
subnormal ones are normal float32 significands too) cover s.
"""
from fractions import Fraction

import numpy as np


def _rn32(x):
    """Round a rational to the nearest float32 (ties to even), normal range."""
    if x == 0:
        return Fraction(0)
    sign = 1 if x > 0 else -1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    scale = Fraction(2) ** (23 - e)
    m = a * scale
    fl = m.numerator // m.denominator
    frac = m - fl
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * Fraction(fl) / scale


def test_rn32_helper():
    rng = np.random.default_rng(3)
    for v in rng.standard_normal(200) * 10.0 ** rng.integers(-8, 8, 200):
        f = Fraction(float(v))
        assert float(_rn32(f)) == float(np.float32(v))
    # ties to even
    assert _rn32(Fraction(1) + Fraction(1, 2 ** 24)) == 1
    assert _rn32(Fraction(1) + Fraction(3, 2 ** 24)) == Fraction(1) + Fraction(2, 2 ** 23)


def test_quotient_by_reciprocal_and_fma_is_correctly_rounded():
    # r over all 2^23 float32 significands of [1, 2).  In float64 every
    # intermediate below is exact before its one rounding to float32: r y
    # has 48 bits, the remainder r - q0 L is a small multiple of q0's ulp,
    # and q0 + rem y spans under 50 bits; a float64 quotient r / L rounded
    # to float32 is the correctly rounded quotient (it never lands on a
    # float32 midpoint for odd L).
    r = (np.float32(1.0) + np.arange(2 ** 23, dtype=np.float32) * np.float32(2.0 ** -23)).astype(np.float32)
    r64 = r.astype(np.float64)
    for L in (3, 15, 255):
        y = np.float32(1.0) / np.float32(L)
        ref = (r64 / L).astype(np.float32)
        q0 = (r64 * np.float64(y)).astype(np.float32)
        rem64 = r64 - q0.astype(np.float64) * L
        rem = rem64.astype(np.float32)
        assert np.array_equal(rem.astype(np.float64), rem64)  # the FMA remainder is exact
        q = (q0.astype(np.float64) + rem.astype(np.float64) * np.float64(y)).astype(np.float32)
        assert np.array_equal(q, ref), L
        assert not np.array_equal(q0, ref)  # the correction is needed
        # spot checks of the float64 shortcut against exact rationals
        for i in np.random.default_rng(L).integers(0, 2 ** 23, 64):
            fr = Fraction(float(r[i]))
            fy = Fraction(float(y))
            e_q0 = _rn32(fr * fy)
            e_rem = _rn32(fr - e_q0 * L)
            assert _rn32(e_q0 + e_rem * fy) == _rn32(fr / L) == Fraction(float(q[i]))


def test_reciprocal_by_one_newton_step_is_correctly_rounded():
    # every fp16 significand m / 1024, m = 1024..2047, and every float32 y0
    # within one ulp of 1 / s
    checked = 0
    for m in range(1024, 2048):
        s = Fraction(m, 1024)
        exact = 1 / s
        ref = _rn32(exact)
        r32 = np.float32(float(ref))
        ulp = Fraction(float(np.spacing(r32)))
        for c in (np.nextafter(r32, np.float32(0)), r32, np.nextafter(r32, np.float32(np.inf))):
            y0 = Fraction(float(c))
            if abs(y0 - exact) > ulp:
                continue
            e = _rn32(1 - s * y0)
            y = _rn32(y0 + e * y0)
            assert y == ref, (m, float(c))
            checked += 1
    assert checked >= 2048


def _f64_chunk_sums(h16):
    """The running-mode chunk sums as the key statistics kernel forms them in
    float64: k (the fp16 key), h = trunc(16 k), r = k - h / 16, then sum k,
    sum h^2, sum h r and sum r^2 by float64 adds and fused multiply-adds,
    scaled at the end to the integers sum a = 2^24 sum k, sum h l = 2^24
    sum h r and sum l^2 = 2^48 sum r^2 (a = k 2^24 = h 2^20 + l), and the
    128-bit s2 = hh 2^40 + hl 2^21 + ll.  numpy's float64 add and multiply
    round like the kernel's; every product and every partial sum here is
    an exact float64 (below 2^45 of its unit: 1, 2^-24 or 2^-48), so the
    separate multiply and add below equal the kernel's FMAs."""
    k = h16.view(np.float16).astype(np.float64)
    h = np.trunc(k * 16.0)
    r = k - h * 0.0625
    s1 = hh = hl = ll = 0.0
    for i in range(len(k)):
        s1 += k[i]
        hh += h[i] * h[i]
        hl += h[i] * r[i]
        ll += r[i] * r[i]
    s1, hl, ll = s1 * 2.0 ** 24, hl * 2.0 ** 24, ll * 2.0 ** 48
    assert s1 == int(s1) and hh == int(hh) and hl == int(hl) and ll == int(ll)
    return int(s1), (int(hh) << 40) + (int(hl) << 21) + int(ll), (h, r * 2.0 ** 24)


def test_running_chunk_sums_in_float64_are_exact():
    # against exact integer sums of a and a^2 (a = k 2^24) for 32-term chunks
    # (one lane's terms of one channel): random keys of every magnitude,
    # the largest values, mixed signs and subnormals
    rng = np.random.default_rng(11)
    finite = np.arange(0x10000, dtype=np.uint32)
    finite = finite[(finite & 0x7C00) != 0x7C00].astype(np.uint16)  # every finite fp16
    chunks = [rng.choice(finite, 32) for _ in range(400)]
    chunks.append(np.full(32, 0x7BFF, np.uint16))  # 65504 everywhere
    chunks.append(np.full(32, 0xFBFF, np.uint16))  # -65504 everywhere
    chunks.append(np.array([0x7BFF, 0xFBFF] * 16, np.uint16))
    chunks.append(np.arange(1, 33, dtype=np.uint16))  # subnormals
    chunks.append(np.array([0x8000, 0x0000] * 16, np.uint16))  # signed zeros
    for c in chunks:
        s1, s2, (h, l) = _f64_chunk_sums(c)
        ints = [int(Fraction(float(v)) * 2 ** 24) for v in c.view(np.float16)]
        assert s1 == sum(ints)
        assert s2 == sum(v * v for v in ints)
        assert np.all(np.abs(h) < 2 ** 20) and np.all(np.abs(l) < 2 ** 20) and np.all(h * l >= 0)
