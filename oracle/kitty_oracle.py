"""Plain, slow, CPU reference of the Kitty 2-bit KV cache hot path.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources, cited by name throughout:

* [Kitty] "Kitty: Accurate and Efficient 2-bit KV Cache Quantization with
  Dynamic Channel-wise Precision Boost" (arXiv 2511.18643), Abstract: Key
  channels are ranked by sensitivity and a small fraction is kept at higher
  precision; each mixed-precision Key page is decomposed into two tensors of
  uniform 2-bit precision inside a page-centric KV layout.
* [Velox] VeloxQuant-MLX documentation, "Kitty -- Dynamic Channel-wise
  Mixed-Precision Keys": section "How it works / Prefill phase" steps 1-3
  (per-channel variance over the token axis, top hi_fraction x D channels at
  hi_bit = 4, the rest at lo_bit = 2, asymmetric min/max groups of
  group_size = 32 tokens), section "Effective bit-width" (avg_bits formula),
  table "Tuning avg_bits".  Two bit-width pairs are built: (hi_bit, lo_bit)
  = (4, 2), the default, and (8, 4), the table's last row; ``lo_bit`` names
  the pair (hi_bit = 2 lo_bit, so a boosted code splits into two lo_bit
  planes exactly like the default's).

Arithmetic conventions (readings of points the pages leave open):

* every float32 operation is a separate IEEE round-to-nearest-even op (numpy
  float32 arithmetic; no fused multiply-add, denormals kept);
* ``f16`` is float32 -> float16 round-to-nearest-even, ``f32`` exact widening;
* the per-page channel statistics use a fixed balanced pairwise tree over the
  32 tokens in natural order (``tree32``), never ``np.sum``/``np.var``, whose
  orders are unspecified;
* quantization: step s16 = f16((max - min) / L) with a correctly rounded fp32
  division; codes q = clamp(rne((x - min) * (1 / s)), 0, L) with one fp32
  reciprocal per group; a zero step gives all-zero codes.

Ranking modes.  "page" (the default) ranks each page by its own variance.
"running" follows [Velox] "How it works": Prefill step 1 ranks a head's
channels by their variance over the whole prefill sequence, and the Decode
phase (steps 1-2) re-derives the ranking from running sums of k and k^2.
Sealed pages cannot change afterwards, so a page takes the ranking current
when it is sealed: the prefill ranking for prefill pages, the running one
over all tokens stored so far for a page sealed by an append.  The sums are
kept exactly (integers in units of 2^-24 and 2^-48; ``fixed24``), and the
score n * sum(k^2) - (sum k)^2 (n^2 times the population variance of the
formula in Decode step 2) is exact, so its value does not depend on the
order of accumulation.
"""
from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 128          # D, the head dimension every page record assumes
PAGE_TOKENS = 32        # tokens per page = Key group size ([Velox] group_size)
V_GROUP = 32            # channels per Value group (one fp16 scale/min each)
LO_LEVELS = 3           # 2-bit codes 0..3 ([Velox] lo_bit = 2)
HI_LEVELS = 15          # 4-bit codes 0..15 ([Velox] hi_bit = 4)
LO_BITS = (2, 4)        # supported lo_bit; hi_bit = 2 * lo_bit ("Tuning avg_bits": (4, 2) and (8, 4))


def levels(lo_bit):
    """(lo, hi) level counts of a bit-width pair: 2^lo_bit - 1, 2^(2 lo_bit) - 1."""
    if lo_bit not in LO_BITS:
        raise ValueError("lo_bit must be 2 or 4")
    return (1 << lo_bit) - 1, (1 << (2 * lo_bit)) - 1

_F32 = np.float32
_F16 = np.float16


def f16(x):
    """float32 -> float16, round to nearest even."""
    return np.asarray(x, _F32).astype(_F16)


def f32(x):
    """Exact widening to float32."""
    return np.asarray(x).astype(_F32)


def f32_stat(x):
    """fp16 input widened to float32 with -0 read as +0, so that a page's
    minimum (and the stored fp16 minimum) has a unique sign."""
    return (np.asarray(x).astype(_F32) + _F32(0.0)).astype(_F32)


# --------------------------------------------------------------------------
# Key page: statistics, ranking, codes, two-plane decomposition
# --------------------------------------------------------------------------

def tree32(a, axis=-2):
    """Balanced pairwise float32 sum of 32 entries along ``axis``:
    five levels, a'_j = a_2j + a_(2j+1), each add rounded to float32."""
    a = np.moveaxis(np.asarray(a, _F32), axis, 0)
    if a.shape[0] != PAGE_TOKENS:
        raise ValueError("tree32 needs 32 entries")
    while a.shape[0] > 1:
        a = (a[0::2] + a[1::2]).astype(_F32)
    return a[0]


def page_stats(x):
    """Per-channel statistics of one Key page ([Velox] Prefill step 1: the
    variance of each channel over the token axis; [Kitty] ranks channels by
    this sensitivity).

    x: float32 [..., 32, D] (values of fp16 keys).  Returns (mu, m2, mn, mx),
    each [..., D]: mean = tree32(x) / 32, m2 = tree32((x - mu)^2) (the
    population variance times 32), and the exact min and max."""
    x = np.asarray(x, _F32)
    mu = (tree32(x, -2) * _F32(1.0 / PAGE_TOKENS)).astype(_F32)
    d = (x - mu[..., None, :]).astype(_F32)
    e = (d * d).astype(_F32)
    m2 = tree32(e, -2)
    return mu, m2, x.min(axis=-2), x.max(axis=-2)


def rank_channels(m2, n_hi):
    """Dynamic Channel-wise Precision Boost selection ([Kitty] Abstract;
    [Velox] Prefill step 2): the n_hi channels with the largest m2, ties
    to the lower channel index.  Returns (idx, mask): idx [..., n_hi] uint8
    ascending, mask [..., D] bool."""
    m2 = np.asarray(m2, _F32)
    D = m2.shape[-1]
    order = np.argsort(-m2, axis=-1, kind="stable")[..., :n_hi]
    idx = np.sort(order, axis=-1)
    mask = np.zeros(m2.shape, bool)
    if n_hi:
        np.put_along_axis(mask, idx, True, axis=-1)
    if D > 256:
        raise ValueError("uint8 channel index needs D <= 256")
    return idx.astype(np.uint8), mask


RANK_MODES = ("page", "running")


def fixed24(k16):
    """fp16 values as exact integers in units of 2^-24 (every fp16 value is a
    multiple of 2^-24 below 2^16): Python ints in an object array."""
    a = np.asarray(k16, _F16).astype(np.float64) * 2.0 ** 24     # exact, |a| < 2^40
    return a.astype(np.int64).astype(object)


def running_scores(s1, s2, n):
    """Exact running-variance score per channel ([Velox] Decode phase step
    2): with s1 = sum a, s2 = sum a^2 over n tokens (a = fixed24(k)),
    n * s2 - s1^2 = n^2 * (sum k^2 / n - (sum k / n)^2) in units of 2^-48."""
    return n * s2 - s1 * s1


def rank_scores(scores, n_hi):
    """The n_hi channels with the largest exact score, ties to the lower
    channel index (the same rule as rank_channels).  scores: object array
    [..., D] of Python ints.  Returns (idx uint8 ascending, mask bool)."""
    sc = np.asarray(scores, object)
    D = sc.shape[-1]
    flat = sc.reshape(-1, D)
    mask = np.zeros(flat.shape, bool)
    for r in range(flat.shape[0]):
        order = sorted(range(D), key=lambda c: (-flat[r, c], c))[:n_hi]
        mask[r, order] = True
    mask = mask.reshape(sc.shape)
    idx = np.nonzero(mask.reshape(-1, D))[1].reshape(sc.shape[:-1] + (n_hi,)).astype(np.uint8)
    return idx, mask


def quantize_levels(x, mn, mx, levels):
    """Asymmetric min/max quantization of x onto {0..levels} ([Velox] Prefill
    step 3).  x, mn, mx: float32, broadcastable; levels: int, broadcastable.
    Returns (codes uint8 shaped like x, s16 float16 shaped like mn)."""
    x = np.asarray(x, _F32)
    mn = np.asarray(mn, _F32)
    mx = np.asarray(mx, _F32)
    L = np.asarray(levels, _F32)
    r = (mx - mn).astype(_F32)
    s16 = f16((r / L).astype(_F32))
    s = f32(s16)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.where(s != 0, (_F32(1.0) / s).astype(_F32), _F32(0.0)).astype(_F32)
        t = ((x - mn).astype(_F32) * inv).astype(_F32)
    q = np.clip(np.rint(t), 0, L).astype(np.uint8)
    q = np.where(s != 0, q, np.uint8(0)).astype(np.uint8)
    return q, np.broadcast_to(s16, np.broadcast_shapes(s16.shape, mn.shape)).astype(_F16)


def quant_k_page(k16, n_hi, lo_bit=2, mask=None):
    """Quantize Key pages.  k16: fp16 [..., 32, D]; n_hi boosted channels;
    lo_bit 2 (hi_bit 4) or 4 (hi_bit 8); ``mask`` (optional, bool
    broadcastable to [..., D] with n_hi True per row) gives the boosted
    channels instead of the page's own ranking (the "running" mode).

    Returns a dict with the direct codes ``q`` (hi_bit on boosted channels,
    lo_bit elsewhere) and the two uniform lo_bit tensors of the decomposition
    ([Kitty] Abstract): ``base`` [..., 32, D] = q >> lo_bit on boosted
    channels, q elsewhere; ``boost`` [..., 32, n_hi] = the low lo_bit bits of
    q on the boosted channels listed by ``idx``; ``kscale`` [..., D] fp16 =
    2^lo_bit * step on boosted channels, step elsewhere; ``kmin`` [..., D]
    fp16."""
    lo_l, hi_l = levels(lo_bit)
    x = f32_stat(k16)
    _, m2, mn, mx = page_stats(x)
    if mask is None:
        idx, mask = rank_channels(m2, n_hi)
    else:
        mask = np.broadcast_to(np.asarray(mask, bool), m2.shape)
        D = mask.shape[-1]
        idx = np.nonzero(mask.reshape(-1, D))[1].reshape(mask.shape[:-1] + (n_hi,)).astype(np.uint8)
    lv = np.where(mask, hi_l, lo_l)
    q, s16 = quantize_levels(x, mn[..., None, :], mx[..., None, :], lv[..., None, :])
    s16 = s16[..., 0, :]
    base = np.where(mask[..., None, :], q >> lo_bit, q).astype(np.uint8)
    gather = np.broadcast_to(idx[..., None, :].astype(np.intp), q.shape[:-1] + (n_hi,))
    boost = (np.take_along_axis(q, gather, axis=-1) & lo_l).astype(np.uint8)
    with np.errstate(over="ignore"):   # 2^lo_bit * step is only kept where it fits (boosted channels)
        kscale = np.where(mask, f16(f32(s16) * _F32(1 << lo_bit)), s16).astype(_F16)
    kmin = f16(mn)
    return dict(q=q, m2=m2, mask=mask, idx=idx, step=s16, base=base, boost=boost,
                kscale=kscale, kmin=kmin, lo_bit=lo_bit)


def quant_v_page(v16, lo_bit=2):
    """Quantize Value pages: per token, groups of 32 channels, lo_bit
    asymmetric min/max.  v16: fp16 [..., 32, D].  Returns dict with ``a``
    [..., 32, D] codes, ``vscale``/``vmin`` [..., 32, D/32] fp16."""
    lo_l, _ = levels(lo_bit)
    y = f32_stat(v16)
    shp = y.shape
    yg = y.reshape(shp[:-1] + (shp[-1] // V_GROUP, V_GROUP))
    mn = yg.min(axis=-1)
    mx = yg.max(axis=-1)
    a, s16 = quantize_levels(yg, mn[..., None], mx[..., None], lo_l)
    return dict(a=a.reshape(shp), vscale=s16[..., 0], vmin=f16(mn))


def dequant_k(base, boost, kscale, kmin, idx, lo_bit=2):
    """Dequantized keys k^ [..., 32, D] float32: on boosted channels the full
    code is 2^lo_bit * base + boost at step kscale / 2^lo_bit, elsewhere base
    at step kscale; k^ = f32(code * step + kmin) (one rounding)."""
    n_hi = idx.shape[-1]
    scale = 1 << lo_bit
    qfull = base.astype(np.int32)
    mask = np.zeros(kscale.shape, bool)
    if n_hi:
        gi = np.broadcast_to(idx[..., None, :].astype(np.intp), base.shape[:-1] + (n_hi,))
        hi_base = np.take_along_axis(qfull, gi, axis=-1)
        np.put_along_axis(qfull, gi, scale * hi_base + boost.astype(np.int32), axis=-1)
        np.put_along_axis(mask, idx.astype(np.intp), True, axis=-1)
    ks = f32(kscale)
    s_eff = np.where(mask, (ks * _F32(1.0 / scale)).astype(_F32), ks).astype(_F32)
    prod = (qfull.astype(_F32) * s_eff[..., None, :]).astype(_F32)
    return (prod + f32(kmin)[..., None, :]).astype(_F32)


def dequant_v(a, vscale, vmin):
    """Dequantized values v^ [..., 32, D] float32 = f32(a * vscale + vmin)."""
    rep = a.shape[-1] // vscale.shape[-1]
    s = np.repeat(f32(vscale), rep, axis=-1)
    m = np.repeat(f32(vmin), rep, axis=-1)
    return ((a.astype(_F32) * s).astype(_F32) + m).astype(_F32)


# --------------------------------------------------------------------------
# Byte layout of one page record (one page of 32 tokens x one KV head)
# --------------------------------------------------------------------------
#
# This layout is this library's own design (the pages fix only that a page
# holds two uniform 2-bit Key tensors plus the boosted channel list).  Field
# order and sizes, n = boost slots = n_hi rounded up to a multiple of 16
# (slots n_hi .. n - 1 are padding: boost code 0, index 0; see boost_slots):
#
#   0            K base codes   1024 B   64 chunks x 16 B
#   1024         K boost codes  8n B     (see _boost_words)
#   1024+8n      V codes        1024 B   64 chunks x 16 B
#   2048+8n      kscale         fp16[128], channel order
#   2304+8n      kmin           fp16[128]
#   2560+8n      vscale         fp16[4][32]: [g][kappa] = token tau(kappa)
#   2816+8n      vmin           fp16[4][32]
#   3072+8n      idx            uint8[n], ascending
#   total 3072 + 9n bytes.
#
# Code words.  Every code plane is a sequence of little-endian 32-bit words
# holding 16 two-bit codes for two "combos" A and B of 8 elements e = 0..7:
# element e of combo A sits at bits 16*(e//4) + 4*(e%2) + 2*((e//2)%2),
# element e of combo B 8 bits higher.  So byte 0 holds combo A's elements
# 0..3, byte 1 combo B's 0..3, bytes 2 and 3 their elements 4..7, and each
# nibble's low two bits hold elements 0, 1 (4, 5), its high two bits
# elements 2, 3 (6, 7).  (The layout is this repository's choice; the pages
# give none.)
#
# Chunk c (0..63) of a 16-byte plane is word x = 0..3 at byte 16c + 4x, with
# u = c % 16 and w = c // 16:
#   K base:  combo A element e = token u,      channel 32x + 8w + e
#            combo B element e = token 16 + u, channel 32x + 8w + e
#   V codes: combo A element e = token tau(w, e), channel 16*(2x) + u
#            combo B element e = token tau(w, e), channel 16*(2x+1) + u
# with tau(w, e) = 4w + e // 2 + 16 * (e % 2): value index kappa = 8w + e holds
# token kappa // 2 + 16 * (kappa % 2) (see ``tau``).
#
# The (8, 4) pair (lo_bit 4) uses 4-bit planes of the same shape: a word
# holds one combo of 8 elements, element e at bits 16*(e//4) + 8*(e%2) +
# 4*((e//2)%2) (each byte holds two elements, e and e + 2, in its low and high
# nibble), and
# a chunk has twice the words, combo A at word 2x and combo B at word 2x + 1
# (byte 32c + 4(2x + combo)), with the same tokens and channels as above.
# The boost plane has two words per lane and slot block (byte 8(c*nf + b) +
# 4*combo; a half block at byte 512 nf + 8c + 4*combo for c < 32).  Field
# sizes: K base 2048 B, K boost 16n B, V codes 2048 B, then the same metadata
# and idx: 5120 + 17n bytes.
#
# K boost: nf = n // 32 full slot blocks, then, if n % 32 == 16, one half
# block.  Full block b of chunk c (c = 0..63) is the word at byte 4*(c*nf+b):
# combo A element e = token u, slot 32b + 8w + e; combo B = token 16 + u.
# The half block is the word at byte 256*nf + 4c for c = 0..31, slots
# 32nf + 8w + e.
#
# Value metadata index kappa = 8w + e stands for token tau(w, e).

def boost_slots(n_hi):
    """Boost slots of a record holding n_hi boosted channels: n_hi rounded up
    to a multiple of 16, so the slot blocks keep their shape for any
    hi_fraction; the padding slots hold code 0 and index 0 and stand for no
    channel."""
    return -(-int(n_hi) // 16) * 16


def record_bytes(n_hi, head_dim=HEAD_DIM, lo_bit=2):
    if head_dim != HEAD_DIM:
        raise ValueError("the record layout is defined for head_dim 128")
    if n_hi < 0 or n_hi > head_dim:
        raise ValueError("n_hi must be in 0..head_dim")
    levels(lo_bit)
    n = boost_slots(n_hi)
    return 1024 * lo_bit + 4 * lo_bit * n + 1024 + n


def page_bytes(n_kv_heads, n_hi, lo_bit=2):
    """Bytes of one physical page (all KV heads), padded to 256."""
    raw = n_kv_heads * record_bytes(n_hi, lo_bit=lo_bit)
    return (raw + 255) // 256 * 256


def tau(w, e):
    """Token of value index kappa = 8w + e: kappa 2t holds token t and
    kappa 2t + 1 token t + 16 (t < 16)."""
    w = np.asarray(w)
    e = np.asarray(e)
    return 4 * w + e // 2 + 16 * (e % 2)


def _bitpos(e):
    """Bit of element e (0..7) of combo A in a 2-bit code word (combo B: 8
    higher)."""
    return 16 * (e // 4) + 4 * (e % 2) + 2 * ((e // 2) % 2)


def _word(a8, b8):
    """Pack combos a8, b8 ([..., 8] codes 0..3) into uint32 words."""
    a8 = np.asarray(a8, np.uint32)
    b8 = np.asarray(b8, np.uint32)
    w = np.zeros(a8.shape[:-1], np.uint32)
    for e in range(8):
        sh = _bitpos(e)
        w |= (a8[..., e] & 3) << np.uint32(sh)
        w |= (b8[..., e] & 3) << np.uint32(sh + 8)
    return w


def _unword(w):
    """Inverse of _word: uint32 [...] -> (a8, b8) uint8 [..., 8]."""
    w = np.asarray(w, np.uint32)
    a8 = np.zeros(w.shape + (8,), np.uint8)
    b8 = np.zeros(w.shape + (8,), np.uint8)
    for e in range(8):
        sh = _bitpos(e)
        a8[..., e] = (w >> np.uint32(sh)) & 3
        b8[..., e] = (w >> np.uint32(sh + 8)) & 3
    return a8, b8


_C = np.arange(64)
_U = _C % 16
_W = _C // 16
_E = np.arange(8)


def _bitpos4(e):
    """Bit of element e (0..7) in a 4-bit code word: byte 0 holds elements 0
    (low nibble) and 2 (high), byte 1 elements 1 and 3, bytes 2 and 3
    elements 4, 6 and 5, 7."""
    return 16 * (e // 4) + 8 * (e % 2) + 4 * ((e // 2) % 2)


def _word4(a8):
    """Pack one combo a8 ([..., 8] codes 0..15) into uint32 words: element e
    at bits _bitpos4(e)."""
    a8 = np.asarray(a8, np.uint32)
    w = np.zeros(a8.shape[:-1], np.uint32)
    for e in range(8):
        w |= (a8[..., e] & 15) << np.uint32(_bitpos4(e))
    return w


def _unword4(w):
    """Inverse of _word4: uint32 [...] -> uint8 [..., 8]."""
    w = np.asarray(w, np.uint32)
    a8 = np.zeros(w.shape + (8,), np.uint8)
    for e in range(8):
        a8[..., e] = (w >> np.uint32(_bitpos4(e))) & 15
    return a8


def _kbase_index():
    # [chunk, x, e] -> (token A, token B, channel)
    ch = 32 * np.arange(4)[None, :, None] + 8 * _W[:, None, None] + _E[None, None, :]
    tA = np.broadcast_to(_U[:, None, None], ch.shape)
    return tA, tA + 16, ch


def _vcode_index():
    # [chunk, x, e] -> (token, channel A, channel B)
    tok = np.broadcast_to(tau(_W[:, None, None], _E[None, None, :]), (64, 4, 8))
    chA = np.broadcast_to(16 * (2 * np.arange(4))[None, :, None] + _U[:, None, None], (64, 4, 8))
    return tok, chA, chA + 16


def _boost_slots(n_hi):
    """List of (byte offset array [nw], token A [nw,8], token B, slot [nw,8])."""
    nf = n_hi // 32
    offs, tA, sl = [], [], []
    for c in range(64):
        for b in range(nf):
            offs.append(4 * (c * nf + b))
            tA.append(np.full(8, c % 16))
            sl.append(32 * b + 8 * (c // 16) + _E)
    if n_hi % 32:
        for c in range(32):
            offs.append(256 * nf + 4 * c)
            tA.append(np.full(8, c % 16))
            sl.append(32 * nf + 8 * (c // 16) + _E)
    if not offs:
        return (np.zeros(0, int), np.zeros((0, 8), int), np.zeros((0, 8), int), np.zeros((0, 8), int))
    tA = np.array(tA)
    return np.array(offs), tA, tA + 16, np.array(sl)


def _kappa_tokens():
    kap = np.arange(32)
    return tau(kap // 8, kap % 8)


def _put_plane(out, o, codesA, codesB, lo_bit):
    """Write a 64-chunk code plane at byte o: codesA/codesB [64, 4, 8] (chunk,
    word x, element) -> 2-bit words (16 B per chunk) or 4-bit word pairs
    (32 B per chunk)."""
    if lo_bit == 2:
        words = _word(codesA, codesB)                                # [64, 4]
    else:
        words = np.stack([_word4(codesA), _word4(codesB)], axis=-1)  # [64, 4, 2]
    raw = words.reshape(-1).astype("<u4").view(np.uint8)
    out[o:o + raw.size] = raw
    return o + raw.size


def _get_plane(buf, o, lo_bit):
    """Inverse of _put_plane: (codesA, codesB) [64, 4, 8] and the next offset."""
    if lo_bit == 2:
        n = 1024
        a8, b8 = _unword(buf[o:o + n].view("<u4").reshape(64, 4))
    else:
        n = 2048
        ws = buf[o:o + n].view("<u4").reshape(64, 4, 2)
        a8, b8 = _unword4(ws[..., 0]), _unword4(ws[..., 1])
    return a8, b8, o + n


def _boost_offsets(n_hi, lo_bit):
    """Byte offsets (within the boost plane) of the words of _boost_slots:
    (combo A offsets, combo B offsets); equal for the 2-bit planes, whose
    words hold both combos."""
    offs, _, _, _ = _boost_slots(n_hi)
    if lo_bit == 2:
        return offs, offs
    nf = n_hi // 32
    # 2-bit byte 4*(c*nf + b) -> 4-bit byte 8*(c*nf + b); half block 256nf + 4c -> 512nf + 8c
    o2 = np.asarray(offs)
    oA = np.where(o2 < 256 * nf, 2 * o2, 512 * nf + 2 * (o2 - 256 * nf)) if len(o2) else o2
    return oA, oA + 4


def pack_record(kf, vf):
    """Bytes of one page record (uint8 [record_bytes]) from the logical fields
    of quant_k_page / quant_v_page for a single page (no leading dims); the
    bit-width pair is kf["lo_bit"] (2 if absent).  Padding slots beyond the
    n_hi boosted channels get code 0 and index 0."""
    n_real = kf["idx"].shape[-1]
    n_hi = boost_slots(n_real)
    lo_bit = int(kf.get("lo_bit", 2))
    out = np.zeros(record_bytes(n_real, lo_bit=lo_bit), np.uint8)
    base, a = kf["base"], vf["a"]
    boost = np.zeros((PAGE_TOKENS, n_hi), np.uint8)
    boost[:, :n_real] = kf["boost"]
    idx = np.zeros(n_hi, np.uint8)
    idx[:n_real] = kf["idx"]
    tA, tB, ch = _kbase_index()
    o = _put_plane(out, 0, base[tA, ch], base[tB, ch], lo_bit)
    offs, bA, bB, sl = _boost_slots(n_hi)
    if len(offs):
        oA, oB = _boost_offsets(n_hi, lo_bit)
        if lo_bit == 2:
            bw = _word(boost[bA, sl], boost[bB, sl])
            for off, wv in zip(oA, bw):
                out[o + off:o + off + 4] = np.array([wv], "<u4").view(np.uint8)
        else:
            for offa, offb, wa, wb in zip(oA, oB, _word4(boost[bA, sl]), _word4(boost[bB, sl])):
                out[o + offa:o + offa + 4] = np.array([wa], "<u4").view(np.uint8)
                out[o + offb:o + offb + 4] = np.array([wb], "<u4").view(np.uint8)
    o += 4 * lo_bit * n_hi
    tok, cA, cB = _vcode_index()
    o = _put_plane(out, o, a[tok, cA], a[tok, cB], lo_bit)
    for arr in (kf["kscale"], kf["kmin"]):
        out[o:o + 256] = np.asarray(arr, "<f2").view(np.uint8)
        o += 256
    kt = _kappa_tokens()
    for arr in (vf["vscale"], vf["vmin"]):          # [32 tokens, 4 groups]
        out[o:o + 256] = np.ascontiguousarray(np.asarray(arr, "<f2")[kt, :].T).view(np.uint8).reshape(-1)
        o += 256
    out[o:o + n_hi] = idx
    return out


def unpack_record(buf, n_hi, lo_bit=2):
    """Inverse of pack_record: logical fields from one record's bytes (the
    n_hi boosted channels; padding slots are dropped)."""
    buf = np.asarray(buf, np.uint8)
    if buf.shape[0] != record_bytes(n_hi, lo_bit=lo_bit):
        raise ValueError("record size mismatch")
    n_real, n_hi = n_hi, boost_slots(n_hi)
    base = np.zeros((PAGE_TOKENS, HEAD_DIM), np.uint8)
    tA, tB, ch = _kbase_index()
    a8, b8, o = _get_plane(buf, 0, lo_bit)
    base[tA, ch] = a8
    base[tB, ch] = b8
    boost = np.zeros((PAGE_TOKENS, n_hi), np.uint8)
    offs, bA, bB, sl = _boost_slots(n_hi)
    if len(offs):
        oA, oB = _boost_offsets(n_hi, lo_bit)
        wA = np.array([buf[o + off:o + off + 4].view("<u4")[0] for off in oA], np.uint32)
        if lo_bit == 2:
            a8, b8 = _unword(wA)
        else:
            wB = np.array([buf[o + off:o + off + 4].view("<u4")[0] for off in oB], np.uint32)
            a8, b8 = _unword4(wA), _unword4(wB)
        boost[bA, sl] = a8
        boost[bB, sl] = b8
    o += 4 * lo_bit * n_hi
    a = np.zeros((PAGE_TOKENS, HEAD_DIM), np.uint8)
    tok, cA, cB = _vcode_index()
    a8, b8, o = _get_plane(buf, o, lo_bit)
    a[tok, cA] = a8
    a[tok, cB] = b8
    kscale = buf[o:o + 256].view("<f2").astype(_F16)
    kmin = buf[o + 256:o + 512].view("<f2").astype(_F16)
    o += 512
    kt = _kappa_tokens()
    vs = np.zeros((PAGE_TOKENS, HEAD_DIM // V_GROUP), _F16)
    vm = np.zeros_like(vs)
    vs[kt, :] = buf[o:o + 256].view("<f2").reshape(4, 32).T
    vm[kt, :] = buf[o + 256:o + 512].view("<f2").reshape(4, 32).T
    o += 512
    idx = buf[o:o + n_real].copy()
    boost = boost[:, :n_real].copy()
    return (dict(base=base, boost=boost, kscale=kscale, kmin=kmin, idx=idx, lo_bit=lo_bit),
            dict(a=a, vscale=vs, vmin=vm))


# --------------------------------------------------------------------------
# Paged cache: prefill, append/seal, dequantized view
# --------------------------------------------------------------------------

class OracleCache:
    """Logical paged cache of a batch: per sequence b, sealed pages stored
    as arrays with leading dims [Hkv, P_b], plus an fp16 tail of 32 slots per
    head ([Kitty] Abstract: page-centric layout; the incomplete tail page
    stays fp16 until it fills)."""

    def __init__(self, batch, n_kv_heads, n_hi, head_dim=HEAD_DIM, lo_bit=2, rank_mode="page"):
        record_bytes(n_hi, head_dim, lo_bit)
        if rank_mode not in RANK_MODES:
            raise ValueError("rank_mode must be 'page' or 'running'")
        self.batch, self.n_kv_heads, self.n_hi, self.head_dim = batch, n_kv_heads, n_hi, head_dim
        self.lo_bit = lo_bit
        self.rank_mode = rank_mode
        # running sums of a = fixed24(k) and a^2 per (sequence, head, channel)
        self.s1 = np.zeros((batch, n_kv_heads, head_dim), object)
        self.s2 = np.zeros((batch, n_kv_heads, head_dim), object)
        self.s1[...] = 0
        self.s2[...] = 0
        self.k = [None] * batch      # dict of arrays [Hkv, P, ...]
        self.v = [None] * batch
        self.tail_k = np.zeros((batch, n_kv_heads, PAGE_TOKENS, head_dim), _F16)
        self.tail_v = np.zeros_like(self.tail_k)
        self.seq_len = np.zeros(batch, np.int64)

    def n_pages(self, b):
        return int(self.seq_len[b]) // PAGE_TOKENS

    def add_tokens_to_sums(self, b, k16):
        """Running sums ([Velox] Prefill step 5, Decode step 1): add the
        tokens k16 fp16 [Hkv, T, D] of sequence b (kept in the "running"
        mode only)."""
        if self.rank_mode != "running":
            return
        a = fixed24(k16)
        self.s1[b] = self.s1[b] + a.sum(axis=1)
        self.s2[b] = self.s2[b] + (a * a).sum(axis=1)

    def running_mask(self, b):
        """Boosted channels [Hkv, D] from the running sums over the
        sequence's seq_len[b] tokens."""
        _, mask = rank_scores(running_scores(self.s1[b], self.s2[b], int(self.seq_len[b])), self.n_hi)
        return mask

    def _add_pages(self, b, k16, v16):
        mask = self.running_mask(b)[:, None, :] if self.rank_mode == "running" else None
        kf = quant_k_page(k16, self.n_hi, self.lo_bit, mask=mask)
        vf = quant_v_page(v16, self.lo_bit)
        kf = {key: kf[key] for key in ("base", "boost", "kscale", "kmin", "idx", "q", "mask")}
        if self.k[b] is None:
            self.k[b], self.v[b] = kf, vf
        else:
            self.k[b] = {key: np.concatenate([self.k[b][key], kf[key]], axis=1) for key in kf}
            self.v[b] = {key: np.concatenate([self.v[b][key], vf[key]], axis=1) for key in vf}

    def page_fields(self, b, h, p):
        kf = {key: self.k[b][key][h, p] for key in ("base", "boost", "kscale", "kmin", "idx")}
        kf["lo_bit"] = self.lo_bit
        vf = {key: self.v[b][key][h, p] for key in ("a", "vscale", "vmin")}
        return kf, vf

    def dequant_sequence(self, b):
        """k^, v^ [Hkv, seq_len, D] float32: sealed pages in order, then
        the tail tokens widened from fp16."""
        H, D = self.n_kv_heads, self.head_dim
        P = self.n_pages(b)
        n_tail = int(self.seq_len[b]) - P * PAGE_TOKENS
        ks, vs = [], []
        if P:
            kf, vf = self.k[b], self.v[b]
            kh = dequant_k(kf["base"][:, :P], kf["boost"][:, :P], kf["kscale"][:, :P],
                           kf["kmin"][:, :P], kf["idx"][:, :P], self.lo_bit)
            vh = dequant_v(vf["a"][:, :P], vf["vscale"][:, :P], vf["vmin"][:, :P])
            ks.append(kh.reshape(H, P * PAGE_TOKENS, D))
            vs.append(vh.reshape(H, P * PAGE_TOKENS, D))
        ks.append(f32(self.tail_k[b, :, :n_tail]))
        vs.append(f32(self.tail_v[b, :, :n_tail]))
        return np.concatenate(ks, axis=1), np.concatenate(vs, axis=1)


def quantize_pages(k, v, n_hi, batch_lens=None, lo_bit=2, rank_mode="page"):
    """Prefill: split fp16 k, v [B, Hkv, S, D] into P = floor(S/32) sealed
    pages and an fp16 tail of S mod 32 tokens ([Velox] Prefill steps 1-3 per
    page of group_size tokens).  ``batch_lens`` (optional, per sequence)
    quantizes only the first len_b tokens of sequence b; ``lo_bit`` picks the
    bit-width pair (2: hi 4 / lo 2, 4: hi 8 / lo 4).  ``rank_mode``
    "running": every page of sequence b takes the ranking by the exact
    variance over all len_b prefill tokens (tail included), and the running
    sums start from those tokens."""
    B, H, S, D = k.shape
    cache = OracleCache(B, H, n_hi, D, lo_bit, rank_mode)
    for b in range(B):
        n = S if batch_lens is None else int(batch_lens[b])
        P = n // PAGE_TOKENS
        cache.add_tokens_to_sums(b, k[b, :, :n])
        cache.seq_len[b] = n
        if P:
            kp = k[b, :, :P * PAGE_TOKENS].reshape(H, P, PAGE_TOKENS, D)
            vp = v[b, :, :P * PAGE_TOKENS].reshape(H, P, PAGE_TOKENS, D)
            cache._add_pages(b, kp, vp)
        t = n - P * PAGE_TOKENS
        cache.tail_k[b, :, :t] = k[b, :, P * PAGE_TOKENS:n]
        cache.tail_v[b, :, :t] = v[b, :, P * PAGE_TOKENS:n]
    return cache


def append_token(cache, k_new, v_new):
    """Decode-time append of one token per sequence (k_new, v_new fp16
    [B, Hkv, D]): store into tail slot n mod 32; when that slot is the 32nd,
    the tail is quantized as page n div 32 exactly like a prefill page and
    the tail becomes empty.  In the "running" mode the token first joins the
    running sums, and a sealed page takes the ranking over all n + 1 tokens."""
    for b in range(cache.batch):
        n = int(cache.seq_len[b])
        slot = n % PAGE_TOKENS
        cache.tail_k[b, :, slot] = k_new[b]
        cache.tail_v[b, :, slot] = v_new[b]
        cache.add_tokens_to_sums(b, k_new[b][:, None, :])
        cache.seq_len[b] = n + 1
        if slot == PAGE_TOKENS - 1:
            cache._add_pages(b, cache.tail_k[b][:, None], cache.tail_v[b][:, None])
    return cache


# --------------------------------------------------------------------------
# Decode attention over the dequantized cache
# --------------------------------------------------------------------------

def softmax_scale(head_dim=HEAD_DIM):
    """float32(1/sqrt(D)): 0.088388346 for D = 128."""
    return _F32(1.0 / math.sqrt(head_dim))


def attention_f32(q, khat, vhat):
    """One decode query per head over all stored tokens, float32.

    q: fp16 [Hq, D]; khat, vhat: float32 [Hkv, S, D].  Query head hq reads
    KV head hq // (Hq / Hkv).  s_t = f32(1/sqrt(D)) * (q . k^_t); p =
    softmax(s) with max subtraction; o = sum_t p_t v^_t.  Returns float32
    [Hq, D]; zeros when S == 0."""
    Hq, D = q.shape
    Hkv, S, _ = khat.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D), _F32)
    if S == 0:
        return out
    sc = softmax_scale(D)
    for hq in range(Hq):
        h = hq // G
        s = ((khat[h] @ f32(q[hq])).astype(_F32) * sc).astype(_F32)
        p = np.exp((s - s.max()).astype(_F32)).astype(_F32)
        out[hq] = ((p @ vhat[h]).astype(_F32) / p.sum(dtype=_F32)).astype(_F32)
    return out


def attention_f64(q, khat, vhat):
    """Same as attention_f32 in float64 (self-check of the float32 one)."""
    Hq, D = q.shape
    Hkv, S, _ = khat.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D), np.float64)
    if S == 0:
        return out
    sc = 1.0 / math.sqrt(D)
    kd = khat.astype(np.float64)
    vd = vhat.astype(np.float64)
    for hq in range(Hq):
        h = hq // G
        s = (kd[h] @ q[hq].astype(np.float64)) * sc
        p = np.exp(s - s.max())
        out[hq] = (p @ vd[h]) / p.sum()
    return out


def decode_attention(cache, q, precision="f32", heads=None, max_len=None):
    """Decode attention for every sequence of the cache: q fp16 [B, Hq, D]
    -> float32 [B, Hq, D].  ``heads`` (optional) restricts to a list of
    KV heads; the other outputs stay zero.  ``max_len`` (optional) bounds
    the tokens attended: the first min(seq_len, max_len) of each sequence."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D), _F32 if precision == "f32" else np.float64)
    G = Hq // cache.n_kv_heads
    fn = attention_f32 if precision == "f32" else attention_f64
    for b in range(B):
        kh, vh = cache.dequant_sequence(b)
        if max_len is not None:
            kh, vh = kh[:, :max_len], vh[:, :max_len]
        hs = range(cache.n_kv_heads) if heads is None else heads
        for h in hs:
            out[b, h * G:(h + 1) * G] = fn(q[b, h * G:(h + 1) * G], kh[h:h + 1], vh[h:h + 1])
    return out


def avg_code_bits(n_hi, head_dim=HEAD_DIM, lo_bit=2):
    """Code bits per Key element of a page record: the base plane's lo_bit
    bits on every channel plus the boost plane's lo_bit bits on n_hi
    channels, counted from the record layout's plane sizes (metadata
    excluded)."""
    base_bits = 512 * lo_bit * 8
    boost_bits = 4 * lo_bit * n_hi * 8
    return (base_bits + boost_bits) / (PAGE_TOKENS * head_dim)
