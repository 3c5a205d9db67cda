"""Pins for the oracle's rANS coder, frequency normalization and model.

The coder is pinned by exact round trips, by the information content of
the coded symbols (rANS stores -log2(f/M) bits per symbol up to the state
overhead), by the uniform-table case where every symbol costs exactly k
bits, and by the end-state invariant (every decoder ends at L).
"""
import numpy as np
import pytest

import oracle

M = 1 << oracle.PROB_BITS
L = oracle.STATE_L


def random_table(rng, nsym, with_ones=True):
    w = rng.gamma(0.7, size=nsym) + 1e-3
    f = np.maximum(1, np.floor(w / w.sum() * M)).astype(np.int64)
    if with_ones:
        f[rng.integers(nsym, size=max(1, nsym // 4))] = 1
    f[np.argmax(f)] += M - f.sum()
    assert f.min() >= 1 and f.sum() == M
    return f.astype(np.uint32)


def draw(rng, f, n):
    return rng.choice(f.size, size=n, p=f / f.sum()).astype(np.int32)


def bitlen(x):
    return int(x).bit_length()


@pytest.mark.parametrize("nsym,nstates,n", [(2, 1, 1), (5, 1, 1000), (40, 64, 8192), (300, 64, 5000),
                                            (17, 64, 63), (3, 7, 1001)])
def test_round_trip_and_end_state(nsym, nstates, n):
    rng = np.random.default_rng(nsym * 1000 + n)
    f = random_table(rng, nsym, with_ones=nsym > 3)
    syms = draw(rng, f, n)
    states, words = oracle.rans_encode(f, syms, nstates)
    assert all(L <= s < (1 << 27) for s in states)
    dec, final = oracle.rans_decode(f, states, words, n)
    assert np.array_equal(dec, syms)
    assert np.all(final == L)


def test_rare_and_dominant_symbols():
    rng = np.random.default_rng(3)
    f = np.array([1, M - 3, 1, 1], np.uint32)
    syms = np.concatenate([np.full(3000, 1), [0, 2, 3, 0, 3]]).astype(np.int32)
    rng.shuffle(syms)
    states, words = oracle.rans_encode(f, syms, 5)
    dec, final = oracle.rans_decode(f, states, words, syms.size)
    assert np.array_equal(dec, syms) and np.all(final == L)


@pytest.mark.parametrize("k", [1, 3, 6, 10])
def test_uniform_table_costs_exactly_k_bits(k):
    """f = M / 2^k for 2^k symbols: each symbol inserts exactly k bits, so
    16 * words + sum(bitlen(x0) - bitlen(L)) == n * k exactly.  A stream
    stores each start state in bitlen(x0) - 1 bits, so a state's stored bits
    are exactly 11 + (its symbols) * k."""
    rng = np.random.default_rng(k)
    f = np.full(1 << k, M >> k, np.uint32)
    for nstates in (1, 64):
        n = 4096
        syms = rng.integers(0, 1 << k, size=n).astype(np.int32)
        states, words = oracle.rans_encode(f, syms, nstates)
        total = 16 * words.size + sum(bitlen(s) - bitlen(L) for s in states)
        assert total == n * k
        dec, _ = oracle.rans_decode(f, states, words, n)
        assert np.array_equal(dec, syms)


def test_state_absorbs_under_16_bits_without_a_word():
    """A state whose symbols carry fewer than 16 bits in total emits no word:
    its start state holds their information (log2 x0 - log2 L equals it up
    to the coder's rounding), which the stream stores at its bit length; past
    16 bits the first word appears.  This is what makes a state's cost its
    information plus a constant (the rate estimate's 18.5 bits)."""
    f = np.array([M - 8, 8], np.uint32)  # symbol 1 carries 7 bits, symbol 0 about 0.01
    for ones in (0, 1, 2):
        syms = np.zeros(128, np.int32)
        syms[:ones] = 1
        info = float(np.sum(np.log2(M / f[syms].astype(np.float64))))
        states, words = oracle.rans_encode(f, syms, 1)
        assert words.size == 0
        # near L = 2^11 the state's integer steps are coarse: 128 symbols of
        # probability 1016/1024 move it by 1.23 bits for their 1.45
        assert abs(np.log2(float(states[0])) - np.log2(L) - info) < 0.25
    syms = np.zeros(128, np.int32)
    syms[:3] = 1  # about 22.4 bits: one word, the rest in the state
    states, words = oracle.rans_encode(f, syms, 1)
    assert words.size == 1
    assert abs(16 + np.log2(float(states[0])) - np.log2(L) - 22.414) < 0.25


def test_size_matches_information():
    """16W + sum(log2 x0) - nstates*log2 L equals sum -log2(f/M) up to the
    coder's small approximation loss (well under 0.5%)."""
    rng = np.random.default_rng(5)
    for nsym in (8, 60, 200):
        f = random_table(rng, nsym)
        n = 200_000
        syms = draw(rng, f, n)
        info = float(np.sum(np.log2(M / f[syms].astype(np.float64))))
        states, words = oracle.rans_encode(f, syms, 64)
        stored_info = 16 * words.size + float(np.sum(np.log2(states.astype(np.float64)))) - 64 * np.log2(L)
        assert stored_info >= info - 64
        assert stored_info <= info * 1.005 + 64, (stored_info, info)


def test_normalize_properties():
    rng = np.random.default_rng(6)
    for _ in range(200):
        n = int(rng.integers(2, 400))
        c = rng.integers(0, 5000, size=n).astype(np.uint64)
        c[rng.integers(n, size=n // 3)] = 0
        c[0] = max(int(c[0]), 1)
        c[-1] = max(int(c[-1]), 1)
        f = oracle.normalize(c)
        used = c > 0
        if used.sum() == 1:
            continue
        assert f.size == n
        assert int(f.sum()) == M
        assert np.all((f > 0) == used)
        assert f.max() <= M - 1


def test_normalize_closed_forms():
    # counts already proportional to M: f = counts / 3 exactly
    c = np.array([M // 2, M // 4, M // 8, M // 8], np.uint64) * 3
    assert np.array_equal(oracle.normalize(c), (c // 3).astype(np.uint32))
    # single used symbol: f = M - 1 plus a never-used companion with f = 1
    assert np.array_equal(oracle.normalize(np.array([7], np.uint64)), np.array([M - 1, 1], np.uint32))
    # a rare symbol keeps f = 1; the deficit goes to the most frequent symbol
    f = oracle.normalize(np.array([1, 10_000_000], np.uint64))
    assert f.tolist() == [1, M - 1]
    # worked by hand (M = 1024): counts [1,1,1,1,1,1,3], N = 9:
    # floor((1*1024 + 4) / 9) = 114, floor((3*1024 + 4) / 9) = 341, sum 1025;
    # the surplus of one comes off the largest frequency
    f = oracle.normalize(np.array([1, 1, 1, 1, 1, 1, 3], np.uint64))
    assert f.tolist() == [114] * 6 + [340]
    # counts [1,1,1], N = 3: floor(1025 / 3) = 341 each, sum 1023; the deficit of
    # one goes to the most frequent symbol, lowest index on a tie
    f = oracle.normalize(np.array([1, 1, 1], np.uint64))
    assert f.tolist() == [342, 341, 341]


def e8_member(v):
    v = np.asarray(v, np.int64)
    par = v & 1
    return par.min() == par.max() and int(((v - par) // 2).sum()) % 2 == 0


def test_model_contexts():
    """Contexts: F for v0; C_b for coordinates 1..6; E_{b,p} for coordinate 7
    with p the parity of z0..z6.  The symbol for coordinate 7 halves the
    range because E8 fixes z7's parity."""
    rng = np.random.default_rng(7)
    for _ in range(3000):
        v = oracle.e8_nearest(rng.normal(0, 3, 8))
        assert e8_member(v)
        ctx, sym = oracle.vector_symbols(v)
        b = int(v[0]) & 1
        z = (v.astype(np.int64) - b) // 2
        p = int(z[:7].sum()) & 1
        assert ctx.tolist() == [0] + [1 + b] * 6 + [3 + 2 * b + p]
        assert sym[0] == v[0]
        assert np.array_equal(sym[1:7], z[1:7])
        assert 2 * sym[7] + p == z[7]
