"""Pins of the K/V gather/scatter oracle against what the definition fixes:
element-by-element brute force over an explicit concatenation, identity and
reversal permutations, round trips, and out-of-range indices."""
import numpy as np
import pytest

from oracle import kvsel

DTYPES = [np.uint16, np.float32]   # bf16 bit patterns, float32


def segments(rng, lens, H_kv, d, dtype):
    if dtype == np.uint16:
        mk = lambda n: rng.integers(0, 1 << 16, size=(H_kv, n, d), dtype=np.uint64).astype(np.uint16)
    else:
        mk = lambda n: rng.standard_normal((H_kv, n, d)).astype(np.float32)
    return [mk(n) for n in lens], [mk(n) for n in lens]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("lens", [[3, 0, 5, 2], [1], [0, 0, 4], [2, 2, 2, 2, 2]])
def test_gather_brute_force(dtype, lens):
    rng = np.random.default_rng(sum(lens) * 7 + len(lens))
    H_kv, d = 2, 3
    K, V = segments(rng, lens, H_kv, d, dtype)
    N = sum(lens)
    Kc, Vc = np.concatenate(K, axis=1), np.concatenate(V, axis=1)
    idx = list(rng.permutation(N)[: max(1, N // 2)]) + [N, -1]
    Ks, Vs = kvsel.gather_kv(K, V, lens, idx)
    for h in range(H_kv):
        for j, i in enumerate(idx):
            for t in range(d):
                ek = Kc[h][i][t] if 0 <= i < N else 0
                ev = Vc[h][i][t] if 0 <= i < N else 0
                assert Ks[h][j][t] == ek and Vs[h][j][t] == ev


@pytest.mark.parametrize("dtype", DTYPES)
def test_identity_and_reversal(dtype):
    rng = np.random.default_rng(3)
    lens = [5, 0, 7, 1, 3]
    K, V = segments(rng, lens, 3, 4, dtype)
    N = sum(lens)
    Kc, Vc = np.concatenate(K, axis=1), np.concatenate(V, axis=1)
    Ks, Vs = kvsel.gather_kv(K, V, lens, np.arange(N))
    assert np.array_equal(Ks, Kc) and np.array_equal(Vs, Vc)
    Ks, Vs = kvsel.gather_kv(K, V, lens, np.arange(N)[::-1])
    assert np.array_equal(Ks, Kc[:, ::-1]) and np.array_equal(Vs, Vc[:, ::-1])


@pytest.mark.parametrize("dtype", DTYPES)
def test_round_trip_and_scatter(dtype):
    rng = np.random.default_rng(4)
    lens = [4, 6, 0, 5]
    K, V = segments(rng, lens, 2, 8, dtype)
    N = sum(lens)
    idx = rng.permutation(N)[:7]
    # scatter(gather(idx)) changes nothing
    K2, V2 = [k.copy() for k in K], [v.copy() for v in V]
    kvsel.scatter_kv(K2, V2, lens, idx, *kvsel.gather_kv(K, V, lens, idx))
    assert all(np.array_equal(a, b) for a, b in zip(K + V, K2 + V2))
    # new rows land at the selected positions only
    Kn, Vn = segments(rng, [len(idx)], 2, 8, dtype)
    Kn, Vn = Kn[0], Vn[0]
    kvsel.scatter_kv(K2, V2, lens, list(idx) + [N, -5], np.concatenate([Kn, Kn[:, :2]], axis=1),
                     np.concatenate([Vn, Vn[:, :2]], axis=1))
    Kc, K2c = np.concatenate(K, axis=1), np.concatenate(K2, axis=1)
    Vc, V2c = np.concatenate(V, axis=1), np.concatenate(V2, axis=1)
    expect_k, expect_v = Kc.copy(), Vc.copy()
    expect_k[:, idx] = Kn
    expect_v[:, idx] = Vn
    assert np.array_equal(K2c, expect_k) and np.array_equal(V2c, expect_v)
    Ks, Vs = kvsel.gather_kv(K2, V2, lens, idx)
    assert np.array_equal(Ks, Kn) and np.array_equal(Vs, Vn)


def test_locate_walks_segments_in_order():
    lens = [2, 0, 3]
    got = [kvsel.locate(lens, i) for i in range(-1, 6)]
    assert got == [(-1, -1), (0, 0), (0, 1), (2, 0), (2, 1), (2, 2), (-1, -1)]


@pytest.mark.parametrize("mutant", ["offset_plus_one", "skip_empty_wrong", "last_segment_first"])
def test_pins_catch_planted_mistakes(mutant, monkeypatch):
    """A plausible indexing mistake planted in the oracle makes the
    brute-force pin fail."""
    real = kvsel.locate

    def bad(lens, i):
        c, off = real(lens, i)
        if c < 0:
            return c, off
        if mutant == "offset_plus_one":
            return c, min(off + 1, lens[c] - 1)
        if mutant == "skip_empty_wrong":
            return (c - 1, off) if c > 0 and lens[c - 1] == 0 else (c, off)
        n = len(lens)   # segments taken in reverse order
        rl = list(lens)[::-1]
        c2, off2 = real(rl, i)
        return n - 1 - c2, off2

    monkeypatch.setattr(kvsel, "locate", bad)
    with pytest.raises((AssertionError, IndexError)):
        test_gather_brute_force(np.float32, [3, 0, 5, 2])
