"""CPU model of the boosted-channel selection the GPU quantizer runs (a
wave-wide bitwise search for the n-th largest key, stopped as soon as
exactly n keys reach the threshold found so far, then ties at the threshold
taken in channel order from ballot popcounts), checked against the plain
definition: the n channels with the largest key, ties to the lower channel
index ("Kitty -- Dynamic Channel-wise Mixed-Precision Keys", How it works /
Prefill phase, step 2).

The model mirrors the wave layout: lane l holds the keys of channels 2l and
2l + 1; a ballot is a 64-bit mask over lanes.  Keys are the bit patterns of
non-negative float32 variances (top bit 30) or 128-bit running scores
(searched from their highest set bit)."""
import numpy as np
import pytest


def _ballot(pred):
    """64-bit mask of the lanes whose predicate holds."""
    m = 0
    for lane, p in enumerate(pred):
        if p:
            m |= 1 << lane
    return m


def select_top_model(keys, n, top, rounds=None):
    """Boosted mask [128] from keys [128] (Python ints >= 0) by the GPU's
    algorithm; `rounds` (a list) receives the number of ballot rounds."""
    k0 = [keys[2 * l] for l in range(64)]
    k1 = [keys[2 * l + 1] for l in range(64)]
    T, cnt_t = 0, 128
    bit = top
    while bit >= 0 and cnt_t != n:
        cand = T | (1 << bit)
        cnt = bin(_ballot([x >= cand for x in k0])).count("1") + bin(_ballot([x >= cand for x in k1])).count("1")
        if cnt >= n:
            T, cnt_t = cand, cnt
        bit -= 1
    if rounds is not None:
        rounds.append(top - bit)
    gt = bin(_ballot([x > T for x in k0])).count("1") + bin(_ballot([x > T for x in k1])).count("1")
    e0, e1 = _ballot([x == T for x in k0]), _ballot([x == T for x in k1])
    need = n - gt
    out = np.zeros(128, bool)
    for lane in range(64):
        below = (1 << lane) - 1
        before0 = bin(e0 & below).count("1") + bin(e1 & below).count("1")
        before1 = before0 + ((e0 >> lane) & 1)
        out[2 * lane] = k0[lane] > T or (k0[lane] == T and before0 < need)
        out[2 * lane + 1] = k1[lane] > T or (k1[lane] == T and before1 < need)
    return out


def select_top_definition(keys, n):
    order = sorted(range(128), key=lambda c: (-keys[c], c))
    out = np.zeros(128, bool)
    out[order[:n]] = True
    return out


def _f32_keys(rng, kind):
    if kind == "random":
        x = rng.standard_normal(128).astype(np.float32) ** 2
    elif kind == "few_values":       # heavy ties everywhere
        x = rng.integers(0, 5, 128).astype(np.float32) * np.float32(0.75)
    elif kind == "all_equal":
        x = np.full(128, 1.5, np.float32)
    elif kind == "zeros":
        x = np.zeros(128, np.float32)
    elif kind == "tie_at_boundary":  # distinct large keys, a tied block, small keys
        x = rng.uniform(0.0, 1.0, 128).astype(np.float32)
        perm = rng.permutation(128)
        x[perm[:40]] = rng.uniform(10.0, 20.0, 40).astype(np.float32)
        x[perm[40:80]] = np.float32(5.0)
    elif kind == "subnormal":
        x = (rng.integers(0, 4, 128) * 2.0 ** -140).astype(np.float32)
    return [int(b) for b in x.view(np.uint32)]


@pytest.mark.parametrize("kind", ["random", "few_values", "all_equal", "zeros", "tie_at_boundary", "subnormal"])
def test_float_keys_every_n(kind):
    rng = np.random.default_rng([ord(ch) for ch in kind])
    for trial in range(3):
        keys = _f32_keys(rng, kind)
        for n in range(129):
            assert np.array_equal(select_top_model(keys, n, 30), select_top_definition(keys, n)), (kind, trial, n)


@pytest.mark.parametrize("kind", ["random", "tied", "all_equal", "huge"])
def test_running_score_keys(kind):
    """128-bit scores, searched from the highest set bit of any key (the
    running-mode start bit)."""
    rng = np.random.default_rng(len(kind))
    for trial in range(3):
        if kind == "random":
            keys = [int(rng.integers(0, 2 ** 62)) * int(rng.integers(1, 2 ** 40)) for _ in range(128)]
        elif kind == "tied":
            vals = [int(rng.integers(0, 2 ** 60)) << 50 for _ in range(6)]
            keys = [vals[int(rng.integers(0, 6))] for _ in range(128)]
        elif kind == "all_equal":
            keys = [12345 << 70] * 128
        else:
            keys = [(2 ** 126) - int(rng.integers(0, 3)) for _ in range(128)]
        top = max(max(keys).bit_length() - 1, 0)
        for n in (0, 1, 13, 16, 32, 45, 64, 100, 127, 128):
            assert np.array_equal(select_top_model(keys, n, top), select_top_definition(keys, n)), (kind, trial, n)


def test_early_exit_happens_and_matches_full_search():
    """The early exit fires on distinct keys (fewer ballot rounds than the
    full 31-bit search) and selects the same channels as a search without
    it."""
    rng = np.random.default_rng(7)
    keys = _f32_keys(rng, "random")

    def full(keys, n):
        k = list(keys)
        T = 0
        for bit in range(30, -1, -1):
            cand = T | (1 << bit)
            if sum(x >= cand for x in k) >= n:
                T = cand
        return T

    for n in (1, 13, 32, 100):
        T = full(keys, n)
        assert T == sorted(keys, reverse=True)[n - 1]
        rounds = []
        assert np.array_equal(select_top_model(keys, n, 30, rounds), select_top_definition(keys, n))
        assert rounds[0] < 31, (n, rounds)
