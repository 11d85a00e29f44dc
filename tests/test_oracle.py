"""Pins of the CPU oracle against facts other than itself (CPU only).

Each test names what fixes the expected value: the pages' printed tuning
table, a closed form, exact rational arithmetic (``fractions``), a textbook
special case written independently here, or a float64 brute force.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from mixed_precision_bit_kitty_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng([seed, 4242])


def _page(seed, n_out=4, factor=20.0, lo=0.05, hi=4.0):
    rng = _rng(seed)
    sig = np.exp(rng.uniform(np.log(lo), np.log(hi), 128))
    out = rng.choice(128, n_out, replace=False)
    sig[out] *= factor
    x = (rng.standard_normal((32, 128)) * sig).astype(np.float32).astype(np.float16)
    return x, out


# --------------------------------------------------------------------------
# Bit budget: the pages' tuning table (golden) and closed form
# --------------------------------------------------------------------------

def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "avg_bits_table.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                hf, hb, lb, avg, comp = line.split()
                rows.append((float(hf), int(hb), int(lb), float(avg), float(comp)))
    return rows


def test_avg_bits_golden_table_closed_form():
    # "Effective bit-width": avg_bits = hf*hi_bit + (1-hf)*lo_bit, compression 16/avg.
    rows = _golden_rows()
    assert len(rows) == 4
    for hf, hb, lb, avg, comp in rows:
        assert hf * hb + (1 - hf) * lb == pytest.approx(avg)
        assert 16 / avg == pytest.approx(comp, abs=0.05)


@pytest.mark.parametrize("row", range(3))
def test_record_code_bits_match_golden_table(row):
    # The record's two 2-bit planes carry exactly the printed budget for the
    # (hi_bit 4, lo_bit 2) rows: 2 bits everywhere + 2 more on n_hi channels.
    hf, hb, lb, avg, comp = _golden_rows()[row]
    assert (hb, lb) == (4, 2)
    n_hi = synth.n_hi_for(hf)
    assert O.avg_code_bits(n_hi) == pytest.approx(avg)
    assert 16 / O.avg_code_bits(n_hi) == pytest.approx(comp, abs=0.05)


def test_avg_bits_eighth_fraction():
    # hf = 0.125 (16 channels): 0.125*4 + 0.875*2 = 2.25 bits.
    assert O.avg_code_bits(16) == pytest.approx(2.25)


def test_record_sizes():
    for n in (0, 16, 32, 64, 128):
        assert O.record_bytes(n) == 3072 + 9 * n
        assert O.record_bytes(n) % 16 == 0
    # other widths keep the shape of the next multiple of 16
    for n, slots in ((1, 16), (8, 16), (13, 16), (17, 32), (45, 48), (127, 128)):
        assert O.boost_slots(n) == slots
        assert O.record_bytes(n) == 3072 + 9 * slots
    with pytest.raises(ValueError):
        O.record_bytes(129)
    with pytest.raises(ValueError):
        O.record_bytes(-1)
    assert O.page_bytes(8, 32) == 26880


# --------------------------------------------------------------------------
# Statistics
# --------------------------------------------------------------------------

def _tree_recursive(v):
    # The same balanced tree, written as recursive halving.
    if len(v) == 1:
        return np.float32(v[0])
    h = len(v) // 2
    return np.float32(_tree_recursive(v[:h]) + _tree_recursive(v[h:]))


def test_tree32_order_is_balanced_pairwise():
    rng = _rng(1)
    a = (rng.standard_normal((32, 5)) * np.exp(rng.uniform(-10, 10, (32, 5)))).astype(np.float32)
    t = O.tree32(a, axis=0)
    for j in range(5):
        assert t[j] == _tree_recursive(list(a[:, j]))
    # A different association order gives a different float32 result on
    # such data, so the test above does distinguish orders.
    seq = np.float32(0)
    for v in a[:, 0]:
        seq = np.float32(seq + v)
    assert any(O.tree32(a, 0)[j] != np.float32(np.cumsum(a[:, j], dtype=np.float32)[-1]) for j in range(5))


@pytest.mark.parametrize("seed", range(5))
def test_page_stats_vs_fp64(seed):
    x, _ = _page(seed)
    xf = x.astype(np.float32)
    mu, m2, mn, mx = O.page_stats(xf)
    x64 = xf.astype(np.float64)
    mu64 = x64.mean(axis=0)
    m2_64 = ((x64 - mu64) ** 2).sum(axis=0)
    u = 2.0 ** -24
    assert np.all(np.abs(mu - mu64) <= 8 * u * np.abs(x64).sum(axis=0) / 32)
    # pairwise summation bound (5 levels) plus the rounding of mu and d
    assert np.all(np.abs(m2 - m2_64) <= 16 * u * m2_64 + 1e-30)
    assert np.array_equal(mn, x64.min(0)) and np.array_equal(mx, x64.max(0))
    # population variance: m2 / 32
    assert np.allclose(m2 / 32, x64.var(axis=0), rtol=1e-5)


def test_constant_page_stats():
    x = np.full((32, 128), 0.3, np.float16).astype(np.float32)
    mu, m2, mn, mx = O.page_stats(x)
    assert np.all(m2 == 0) and np.all(mn == mx)


# --------------------------------------------------------------------------
# Ranking
# --------------------------------------------------------------------------

def _rank_bruteforce(m2, k):
    # H = {c : #{c' : m2[c'] > m2[c] or (m2[c'] == m2[c] and c' < c)} < k}
    D = len(m2)
    sel = []
    for c in range(D):
        r = sum(1 for c2 in range(D) if m2[c2] > m2[c] or (m2[c2] == m2[c] and c2 < c))
        if r < k:
            sel.append(c)
    return sel


@pytest.mark.parametrize("k", [0, 16, 32, 64, 128])
def test_rank_bruteforce_and_lexsort(k):
    rng = _rng(7)
    for trial in range(4):
        # heavy ties: few distinct values
        m2 = rng.integers(0, 6 if trial % 2 else 1000, 128).astype(np.float32)
        idx, mask = O.rank_channels(m2, k)
        assert list(idx) == _rank_bruteforce(list(m2), k)
        assert list(idx) == sorted(np.lexsort((np.arange(128), -m2))[:k])
        assert mask.sum() == k and all(mask[i] for i in idx)


def test_rank_all_equal_takes_lowest_indices():
    idx, _ = O.rank_channels(np.ones(128, np.float32), 32)
    assert list(idx) == list(range(32))


def test_rank_matches_fp64_except_near_ties():
    u = 2.0 ** -24
    for seed in range(10):
        x, _ = _page(seed)
        xf = x.astype(np.float32)
        _, m2, _, _ = O.page_stats(xf)
        x64 = xf.astype(np.float64)
        m2_64 = ((x64 - x64.mean(0)) ** 2).sum(0)
        idx, _ = O.rank_channels(m2, 32)
        ref = np.sort(np.argsort(-m2_64, kind="stable")[:32])
        if not np.array_equal(idx, ref):
            # allowed only if the fp64 values at the boundary are within the bound
            kth = np.sort(m2_64)[::-1][31]
            diff = set(idx) ^ set(ref)
            for c in diff:
                assert abs(m2_64[c] - kth) <= 32 * u * kth


def test_planted_outliers_always_selected():
    # Channels whose scale is 20x the largest other scale are boosted
    # ("Evidence": high-variance channels correctly identified).
    for seed in range(20):
        rng = _rng(100 + seed)
        sig = np.exp(rng.uniform(np.log(0.05), np.log(4.0), 128))
        out = rng.choice(128, 8, replace=False)
        sig[out] = sig.max() * 20
        x = (rng.standard_normal((32, 128)) * sig).astype(np.float16)
        kf = O.quant_k_page(x, 32)
        assert set(out) <= set(kf["idx"].tolist())


# --------------------------------------------------------------------------
# Quantization: grid-exact data, exact rational brute force, special cases
# --------------------------------------------------------------------------

def test_grid_exact_two_and_four_bit():
    # x = mn + i*s exactly representable => codes i and exact reconstruction.
    for L, mn, s in ((3, -1.5, 0.25), (15, 1.0, 0.125), (3, 1024.0, 64.0)):
        rng = _rng(L)
        i = rng.integers(0, L + 1, 32)
        i[0], i[1] = 0, L
        x = (mn + i * s).astype(np.float16).astype(np.float32)
        q, s16 = O.quantize_levels(x, x.min(), x.max(), L)
        assert np.array_equal(q, i)
        assert float(s16) == s
        assert np.array_equal(q.astype(np.float32) * np.float32(s16) + np.float32(mn), x)


def _f16_nearest(fr):
    """fp16 value nearest to the Fraction fr (ties to even), by search."""
    v = np.float16(float(fr))
    cands = [np.nextafter(v, np.float16(-np.inf)), v, np.nextafter(v, np.float16(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.array(c).view(np.uint16)) & 1))
    return best


@pytest.mark.parametrize("L", [3, 15])
def test_quantize_bruteforce_fractions(L):
    rng = _rng(11 + L)
    n_checked = n_mid = 0
    for trial in range(200):
        n = 32
        x = (rng.standard_normal(n) * np.exp(rng.uniform(-6, 6))).astype(np.float16)
        xf = x.astype(np.float32)
        q, s16 = O.quantize_levels(xf, xf.min(), xf.max(), L)
        mn = Fraction(float(xf.min()))
        mx = Fraction(float(xf.max()))
        # step: nearest fp16 to the exact (max - min) / L, except double rounding
        exact_step = (mx - mn) / L
        near = _f16_nearest(exact_step)
        if np.float16(s16) != near:
            lo_h = Fraction(float(min(near, np.float16(s16))))
            hi_h = Fraction(float(max(near, np.float16(s16))))
            mid = (lo_h + hi_h) / 2
            assert abs(exact_step - mid) <= exact_step * Fraction(1, 2 ** 23)
            continue
        s = Fraction(float(s16))
        if s == 0:
            assert np.all(q == 0)
            continue
        for xi, qi in zip(xf, q):
            t = (Fraction(float(xi)) - mn) / s
            fl = math.floor(t)
            frac = t - fl
            if abs(frac - Fraction(1, 2)) <= Fraction(2, 2 ** 23) * max(t, 1):
                n_mid += 1          # within rounding of a midpoint: either neighbour
                assert qi in (min(fl, L), min(fl + 1, L))
                continue
            want = fl + (1 if frac > Fraction(1, 2) else 0)
            assert qi == min(max(want, 0), L)
            n_checked += 1
    assert n_checked > 5000 and n_mid < n_checked / 100


def _textbook_per_channel(x, L):
    """Plain per-channel asymmetric min/max quantization over the token axis
    (the hi_fraction = 0 case, KIVI-style Key grouping), float64 division."""
    x = x.astype(np.float64)
    mn = x.min(0)
    mx = x.max(0)
    step = ((mx - mn) / L).astype(np.float16).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(step > 0, (x - mn) / step, 0.0)
    return np.clip(np.rint(t), 0, L), step, t


@pytest.mark.parametrize("n_hi,L", [(0, 3), (128, 15)])
def test_uniform_special_cases_are_textbook(n_hi, L):
    for seed in range(5):
        x, _ = _page(seed)
        kf = O.quant_k_page(x, n_hi)
        want, step, t = _textbook_per_channel(x.astype(np.float32), L)
        near_mid = np.abs(t - np.floor(t) - 0.5) < 1e-5 * np.maximum(t, 1)
        diff = kf["q"] != want
        assert not np.any(diff & ~near_mid)
        assert np.array_equal(kf["step"].astype(np.float64), step)
        if n_hi == 0:
            assert np.array_equal(kf["base"], kf["q"]) and kf["boost"].shape == (32, 0)
        else:
            assert list(kf["idx"]) == list(range(128))
            assert np.array_equal(kf["base"], kf["q"] >> 2)
            assert np.array_equal(kf["boost"], kf["q"] & 3)


def test_constant_channel_codes_zero():
    x, _ = _page(3)
    x[:, 5] = np.float16(-2.75)
    x[:, 77] = np.float16(0.0)
    kf = O.quant_k_page(x, 32)
    assert np.all(kf["q"][:, 5] == 0) and np.all(kf["q"][:, 77] == 0)
    assert kf["kscale"][5] == 0 and kf["kscale"][77] == 0
    kh = O.dequant_k(kf["base"], kf["boost"], kf["kscale"], kf["kmin"], kf["idx"])
    assert np.all(kh[:, 5] == np.float32(-2.75)) and np.all(kh[:, 77] == 0)


def test_tiny_range_subnormal_step():
    # range so small that the step is an fp16 subnormal or zero
    x, _ = _page(4)
    x[:, 9] = np.float16(1.0)
    x[3, 9] = np.nextafter(np.float16(1.0), np.float16(2.0))
    x[:, 10] = np.float16(0.0)
    x[7, 10] = np.float16(2.0 ** -24)
    kf = O.quant_k_page(x, 32)
    for c in (9, 10):
        xs = x[:, c].astype(np.float32)
        s = np.float32(kf["step"][c])
        kh = O.dequant_k(kf["base"], kf["boost"], kf["kscale"], kf["kmin"], kf["idx"])[:, c]
        assert np.all(np.abs(kh - xs) <= max(s, 2.0 ** -24))


def test_boost_plane_reconstructs_exact_4bit_codes():
    for seed in range(5):
        x, _ = _page(seed)
        kf = O.quant_k_page(x, 32)
        kf_all4 = O.quant_k_page(x, 128)
        idx = kf["idx"].astype(int)
        full = (kf["base"][:, idx].astype(int) << 2) | kf["boost"]
        assert np.array_equal(full, kf["q"][:, idx])
        # identical to the direct 4-bit codes of the same channels
        assert np.array_equal(full, kf_all4["q"][:, idx])
        assert np.array_equal(kf["kscale"][idx], (kf_all4["step"][idx].astype(np.float32) * 4).astype(np.float16))


def test_lo_channel_codes_independent_of_boost():
    for seed in range(5):
        x, _ = _page(seed)
        a = O.quant_k_page(x, 32)
        b = O.quant_k_page(x, 0)
        lo = ~a["mask"]
        assert np.array_equal(a["q"][:, lo], b["q"][:, lo])
        assert np.array_equal(a["kscale"][lo], b["kscale"][lo])
        assert np.array_equal(a["kmin"], b["kmin"])


def test_value_groups_textbook():
    rng = _rng(5)
    y = (rng.standard_normal((32, 128)) * np.exp(rng.uniform(-3, 1.4, 128))).astype(np.float16)
    vf = O.quant_v_page(y)
    for t in range(32):
        for g in range(4):
            seg = y[t, 32 * g:32 * g + 32].astype(np.float32)
            want, step, tt = _textbook_per_channel(seg[:, None], 3)
            near_mid = np.abs(tt - np.floor(tt) - 0.5) < 1e-5 * np.maximum(tt, 1)
            got = vf["a"][t, 32 * g:32 * g + 32][:, None]
            assert not np.any((got != want) & ~near_mid)
            assert vf["vscale"][t, g] == np.float16(step[0])
            assert vf["vmin"][t, g] == np.float16(seg.min())
    vh = O.dequant_v(vf["a"], vf["vscale"], vf["vmin"])
    assert np.all(np.abs(vh - y.astype(np.float32)) <= np.repeat(vf["vscale"].astype(np.float32), 32, 1) * 0.5 + 1e-6)


def test_dequant_error_within_half_step():
    for seed in range(5):
        x, _ = _page(seed)
        kf = O.quant_k_page(x, 32)
        kh = O.dequant_k(kf["base"], kf["boost"], kf["kscale"], kf["kmin"], kf["idx"])
        step = kf["step"].astype(np.float32)
        err = np.abs(kh - x.astype(np.float32))
        assert np.all(err <= step * 0.5 * (1 + 2 ** -10) + np.abs(x.astype(np.float32)) * 2 ** -23)


# --------------------------------------------------------------------------
# Error invariants ("Evidence" table of the VeloxQuant page)
# --------------------------------------------------------------------------

def test_hi_channels_lower_normalized_error_than_lo():
    for seed in range(5):
        x, _ = _page(seed)
        xf = x.astype(np.float32)
        kf = O.quant_k_page(x, 32)
        kh = O.dequant_k(kf["base"], kf["boost"], kf["kscale"], kf["kmin"], kf["idx"])
        var = xf.astype(np.float64).var(0)
        nmse = ((kh - xf).astype(np.float64) ** 2).mean(0) / np.maximum(var, 1e-30)
        assert nmse[kf["mask"]].mean() < nmse[~kf["mask"]].mean()


def test_mixed_precision_beats_uniform_2bit_mse():
    for seed in range(5):
        x, _ = _page(seed)
        xf = x.astype(np.float64)
        errs = {}
        for n in (0, 32):
            kf = O.quant_k_page(x, n)
            kh = O.dequant_k(kf["base"], kf["boost"], kf["kscale"], kf["kmin"], kf["idx"])
            errs[n] = ((kh - xf) ** 2).mean(0)
        assert errs[32].sum() < errs[0].sum()
        hi = O.quant_k_page(x, 32)["mask"]
        # per boosted channel the 4-bit grid is not worse than the 2-bit one
        assert np.all(errs[32][hi] <= errs[0][hi] * (1 + 1e-3) + 1e-12)


# --------------------------------------------------------------------------
# Byte layout: explicit positions from the layout description
# --------------------------------------------------------------------------

def _one_code_page(plane, t, c, val, n_hi=32):
    kf = dict(base=np.zeros((32, 128), np.uint8), boost=np.zeros((32, n_hi), np.uint8),
              kscale=np.zeros(128, np.float16), kmin=np.zeros(128, np.float16),
              idx=np.arange(n_hi, dtype=np.uint8))
    vf = dict(a=np.zeros((32, 128), np.uint8), vscale=np.zeros((32, 4), np.float16),
              vmin=np.zeros((32, 4), np.float16))
    {"base": kf["base"], "boost": kf["boost"], "a": vf["a"]}[plane][t, c] = val
    return O.pack_record(kf, vf)[:2048 + 8 * n_hi]      # the three code planes


def test_layout_positions_by_hand():
    # Element e of combo A sits at bit 16*(e//4) + 4*(e%2) + 2*((e//2)%2) of
    # its word, combo B 8 bits higher.
    # base[token 17][channel 42] = 3: token 17 -> combo B, u = 1; channel 42 =
    # 32*1 + 8*1 + 2 -> x = 1, w = 1, e = 2; chunk 16*1 + 1 = 17, word at
    # byte 16*17 + 4 = 276; bit 0 + 8 + 0 + 2 = 10 -> byte 277, bits 2..3.
    r = _one_code_page("base", 17, 42, 3)
    nz = np.nonzero(r)[0]
    assert list(nz) == [277] and r[277] == 3 << 2
    # base[token 4][channel 101] = 2: combo A, u = 4; 101 = 96 + 0 + 5 ->
    # x = 3, w = 0, e = 5; chunk 4, byte 16*4 + 12 = 76; bit 16 + 4 + 0 = 20
    # -> byte 78, bits 4..5.
    r = _one_code_page("base", 4, 101, 2)
    assert list(np.nonzero(r)[0]) == [78] and r[78] == 2 << 4
    # base[token 3][channel 33] = 1: combo A, u = 3; 33 = 32 + 0 + 1 -> x = 1,
    # w = 0, e = 1; chunk 3, byte 16*3 + 4 = 52; bit 0 + 4 + 0 = 4 -> byte 52,
    # bits 4..5.
    r = _one_code_page("base", 3, 33, 1)
    assert list(np.nonzero(r)[0]) == [52] and r[52] == 1 << 4
    # boost (n_hi = 32, one full block) [token 20][slot 9] = 1: combo B, u = 4;
    # slot 9 = 8*1 + 1 -> w = 1, e = 1; chunk 20; word at 1024 + 4*20 = 1104;
    # bit 0 + 8 + 4 + 0 = 12 -> byte 1105, bits 4..5.
    r = _one_code_page("boost", 20, 9, 1)
    assert list(np.nonzero(r)[0]) == [1105] and r[1105] == 1 << 4
    # V codes (n_hi = 32: plane at 1280) a[token 22][channel 53] = 3: token 22 =
    # tau(w=1, e=5) (4 + 2 + 16); channel 53 = 16*3 + 5 -> combo B of x = 1,
    # u = 5; chunk 16 + 5 = 21; word at 1280 + 16*21 + 4 = 1620; bit 16 + 8 +
    # 4 + 0 = 28 -> byte 1623, bits 4..5.
    r = _one_code_page("a", 22, 53, 3)
    assert list(np.nonzero(r)[0]) == [1623] and r[1623] == 3 << 4
    # a[token 7][channel 2] = 1: token 7 = tau(w=1, e=6) (4 + 3); channel 2 ->
    # combo A of x = 0, u = 2; chunk 18; word at 1280 + 16*18 = 1568; bit
    # 16 + 0 + 0 + 2 = 18 -> byte 1570, bits 2..3.
    r = _one_code_page("a", 7, 2, 1)
    assert list(np.nonzero(r)[0]) == [1570] and r[1570] == 1 << 2
    # a[token 17][channel 20] = 2: token 17 = tau(w=0, e=3) (0 + 1 + 16);
    # channel 20 = 16 + 4 -> combo B of x = 0, u = 4; chunk 4; word at
    # 1280 + 16*4 = 1344; bit 0 + 8 + 4 + 2 = 14 -> byte 1345, bits 6..7.
    r = _one_code_page("a", 17, 20, 2)
    assert list(np.nonzero(r)[0]) == [1345] and r[1345] == 2 << 6


def test_layout_half_boost_block():
    # n_hi = 16: a half block only, lanes 0..31; boost[token 3][slot 15]:
    # w = 1, e = 7; chunk 16 + 3 = 19; byte 1024 + 4*19 = 1100; bit 16 + 4 +
    # 2 = 22 -> byte 1102, bits 6..7.
    r = _one_code_page("boost", 3, 15, 2, n_hi=16)
    assert list(np.nonzero(r)[0]) == [1102] and r[1102] == 2 << 6
    # boost[token 16][slot 4]: combo B, u = 0, w = 0, e = 4; chunk 0; byte
    # 1024; bit 16 + 8 + 0 + 0 = 24 -> byte 1027, bits 0..1.
    r = _one_code_page("boost", 16, 4, 3, n_hi=16)
    assert list(np.nonzero(r)[0]) == [1027] and r[1027] == 3


def test_layout_metadata_offsets():
    x, _ = _page(9)
    kf = O.quant_k_page(x, 32)
    vf = O.quant_v_page(x)
    r = O.pack_record(kf, vf)
    o = 1024 + 256 + 1024
    assert np.array_equal(r[o:o + 256].view("<f2"), kf["kscale"])
    assert np.array_equal(r[o + 256:o + 512].view("<f2"), kf["kmin"])
    vs = r[o + 512:o + 768].view("<f2").reshape(4, 32)
    # kappa = 8w + e -> token tau(w, e); kappa 13 = (1, 5) -> token 4 + 2 + 16 = 22,
    # kappa 3 = (0, 3) -> token 1 + 16 = 17, kappa 6 = (0, 6) -> token 3
    assert vs[2, 13] == vf["vscale"][22, 2]
    assert vs[0, 3] == vf["vscale"][17, 0]
    assert vs[1, 6] == vf["vscale"][3, 1]
    assert np.array_equal(r[o + 1024:o + 1056], kf["idx"])


@pytest.mark.parametrize("n_hi", [0, 16, 32, 64, 96, 128])
def test_pack_unpack_roundtrip(n_hi):
    x, _ = _page(n_hi)
    y, _ = _page(n_hi + 1)
    kf = O.quant_k_page(x, n_hi)
    vf = O.quant_v_page(y)
    kf2, vf2 = O.unpack_record(O.pack_record(kf, vf), n_hi)
    for key in kf2:
        assert np.array_equal(kf[key], kf2[key]), key
    for key in vf2:
        assert np.array_equal(vf[key], vf2[key]), key


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _attn_bruteforce(q, kh, vh):
    Hq, D = q.shape
    Hkv, S, _ = kh.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D))
    for hq in range(Hq):
        h = hq // G
        s = [sum(float(q[hq, c]) * float(kh[h, t, c]) for c in range(D)) / math.sqrt(D) for t in range(S)]
        m = max(s)
        p = [math.exp(si - m) for si in s]
        z = sum(p)
        for c in range(D):
            out[hq, c] = sum(p[t] * float(vh[h, t, c]) for t in range(S)) / z
    return out


@pytest.mark.parametrize("S,Hq,Hkv", [(1, 1, 1), (5, 4, 1), (8, 4, 2)])
def test_attention_bruteforce(S, Hq, Hkv):
    rng = _rng(S * 10 + Hq)
    q = rng.standard_normal((Hq, 128)).astype(np.float16)
    kh = (rng.standard_normal((Hkv, S, 128)) * 3).astype(np.float32)
    vh = rng.standard_normal((Hkv, S, 128)).astype(np.float32)
    ref = _attn_bruteforce(q, kh, vh)
    assert np.abs(O.attention_f32(q, kh, vh) - ref).max() < 1e-5
    assert np.abs(O.attention_f64(q, kh, vh) - ref).max() < 1e-12


def test_attention_special_cases():
    rng = _rng(3)
    q = rng.standard_normal((4, 128)).astype(np.float16)
    vh = rng.standard_normal((1, 6, 128)).astype(np.float32)
    kh1 = rng.standard_normal((1, 1, 128)).astype(np.float32)
    assert np.array_equal(O.attention_f32(q, kh1, vh[:, :1]), np.repeat(vh[:, 0], 4, 0))
    khs = np.repeat(kh1, 6, axis=1)
    assert np.allclose(O.attention_f32(q, khs, vh), np.repeat(vh.mean(1), 4, 0), atol=1e-6)
    assert np.all(O.attention_f32(q, khs[:, :0], vh[:, :0]) == 0)


def test_attention_vs_torch_sdpa_on_quantized_cache():
    torch = pytest.importorskip("torch")
    w = synth.TINY
    x = synth.batch(w)
    cache = O.quantize_pages(x["k"], x["v"], w.n_hi)
    kh, vh = cache.dequant_sequence(0)
    out = O.decode_attention(cache, x["q"])[0]
    qt = torch.tensor(x["q"][0].astype(np.float64))[:, None, :]           # [Hq, 1, D]
    kt = torch.tensor(kh.astype(np.float64))
    vt = torch.tensor(vh.astype(np.float64))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0, :].numpy()
    assert np.abs(out - ref).max() < 2e-5


def test_gqa_head_mapping():
    # query head hq reads KV head hq // G (consecutive grouping)
    rng = _rng(8)
    q = rng.standard_normal((8, 128)).astype(np.float16)
    kh = rng.standard_normal((2, 3, 128)).astype(np.float32)
    vh = np.zeros((2, 3, 128), np.float32)
    vh[1] = 1.0
    o = O.attention_f32(q, kh, vh)
    assert np.all(o[:4] == 0) and np.allclose(o[4:], 1.0)


# --------------------------------------------------------------------------
# Cache: prefill, append/seal, determinism
# --------------------------------------------------------------------------

def test_append_stream_equals_prefill():
    w = synth.TINY.with_(n_kv_heads=2, n_q_heads=4)
    x = synth.batch(w, batch=2, ctx=100)
    pre = O.quantize_pages(x["k"], x["v"], 32)
    st = O.OracleCache(2, 2, 32)
    for t in range(100):
        O.append_token(st, x["k"][:, :, t], x["v"][:, :, t])
    assert np.array_equal(pre.seq_len, st.seq_len)
    for b in range(2):
        for key in ("base", "boost", "kscale", "kmin", "idx"):
            assert np.array_equal(pre.k[b][key], st.k[b][key])
        for key in ("a", "vscale", "vmin"):
            assert np.array_equal(pre.v[b][key], st.v[b][key])
        assert np.array_equal(pre.tail_k[b, :, :4], st.tail_k[b, :, :4])
    q = x["q"]
    assert np.array_equal(O.decode_attention(pre, q), O.decode_attention(st, q))


def test_value_bytes_independent_of_boost():
    x, _ = _page(2)
    y, _ = _page(5)
    vf = O.quant_v_page(y)
    r0 = O.pack_record(O.quant_k_page(x, 0), vf)
    r32 = O.pack_record(O.quant_k_page(x, 32), vf)
    assert np.array_equal(r0[1024:2048], r32[1024 + 256:2048 + 256])
    assert np.array_equal(r0[2560:3072], r32[2560 + 256:3072 + 256])


def test_determinism():
    w = synth.TINY
    a = synth.batch(w)
    b = synth.batch(w)
    for key in a:
        assert np.array_equal(a[key], b[key])
    c1 = O.quantize_pages(a["k"], a["v"], 32)
    c2 = O.quantize_pages(b["k"], b["v"], 32)
    assert np.array_equal(O.decode_attention(c1, a["q"]), O.decode_attention(c2, b["q"]))


def test_empty_and_ragged_prefill():
    w = synth.TINY.with_(n_kv_heads=2, n_q_heads=2)
    x = synth.batch(w, batch=3, ctx=70)
    c = O.quantize_pages(x["k"], x["v"], 16, batch_lens=[0, 31, 70])
    assert list(c.seq_len) == [0, 31, 70]
    assert c.n_pages(0) == 0 and c.n_pages(1) == 0 and c.n_pages(2) == 2
    out = O.decode_attention(c, x["q"])
    assert np.all(out[0] == 0)
    kh, vh = c.dequant_sequence(1)
    assert np.array_equal(kh, x["k"][1, :, :31].astype(np.float32))


def test_synth_prefix_property():
    w = synth.LLAMA3_8B
    a = synth.batch(w, batch=2, ctx=64, steps=2)
    b = synth.batch(w, batch=3, ctx=64, steps=2)
    assert np.array_equal(a["k"], b["k"][:2]) and np.array_equal(a["q_new"], b["q_new"][:, :2])
    assert a["k"].dtype == np.float16 and a["k"].shape == (2, 8, 64, 128)
    sk, _ = synth.scales(w)
    assert sk.shape == (8, 128)
    assert all((sk[h] > 4.0).sum() >= 1 for h in range(8))


def test_clamp_when_subnormal_step_rounds_down():
    # (max - min) / L lands between fp16 subnormals and rounds down, so the
    # top value maps past L before clamping: 7 ulp / 3 -> step 2 ulp -> 3.5
    # -> rne 4 -> clamp 3; 21 ulp / 15 -> step 1 ulp -> 21 -> clamp 15.
    ulp = 2.0 ** -24
    for L, top in ((3, 7), (15, 21)):
        x = np.array([0.0, top * ulp, 2 * ulp] + [0.0] * 29, np.float16).astype(np.float32)
        q, s16 = O.quantize_levels(x, x.min(), x.max(), L)
        assert q[1] == L and q.max() == L
        assert float(s16) == (2 * ulp if L == 3 else ulp)


def test_clamp_idle_for_normal_steps():
    # The quantizer kernels leave the clamp out of a page whose steps are all
    # zero or normal fp16 numbers.  That relies on the largest scaled value,
    # (max - min) * (1 / step), staying below L + 1/2, so that round to
    # nearest even never passes L.  It is checked here for every float32
    # significand of max - min in the binade [1, 2), whose steps are normal;
    # the float32 operations and the fp16 rounding of a normal step scale
    # exactly by powers of two, and a random sample over the other binades
    # with normal steps agrees.
    def top_scaled(r, L):
        q = (r / np.float32(L)).astype(np.float32)
        s16 = q.astype(np.float16)
        inv = (np.float32(1.0) / s16.astype(np.float32)).astype(np.float32)
        return (r * inv).astype(np.float32), s16

    r = (np.float32(1.0) + np.arange(2 ** 23, dtype=np.float32) * np.float32(2.0 ** -23)).astype(np.float32)
    rng = np.random.default_rng(0)
    rs = np.ldexp(r[rng.integers(0, 2 ** 23, 1 << 20)], rng.integers(-24, 17, 1 << 20)).astype(np.float32)
    for L in (3, 15, 255):
        t, s16 = top_scaled(r, L)
        assert np.all(np.isfinite(s16)) and np.all(np.abs(s16) >= np.float16(2.0 ** -14))
        assert float(t.max()) < L + 0.5
        t, s16 = top_scaled(rs, L)
        normal = np.isfinite(s16) & (s16 >= np.float16(2.0 ** -14))
        assert normal.sum() > (1 << 19) and float(t[normal].max()) < L + 0.5
        # the oracle's own codes at the top of such ranges stay exact
        for x in (np.array([0.0, 1.0], np.float32), np.array([0.0, 1.9990234], np.float32)):
            q, _ = O.quantize_levels(x, x.min(), x.max(), L)
            assert q.max() == L
    # and a subnormal step does need it (the counterexample above)
    t, _ = top_scaled(np.array([7 * 2.0 ** -24], np.float32), 3)
    assert float(t[0]) >= 3.5


def test_negative_zero_read_as_positive_zero():
    # A page whose minimum is a signed zero stores kmin = +0 (0x0000).
    x = np.abs(_page(6)[0])
    x[:, 3] = np.float16(-0.0)
    x[5, 3] = np.float16(1.0)
    kf = O.quant_k_page(x, 32)
    assert kf["kmin"].view(np.uint16)[3] == 0
    vf = O.quant_v_page(x)
    rows = [t for t in range(32) if t != 5]
    assert np.all(vf["vmin"].view(np.uint16)[rows, 0] == 0)
