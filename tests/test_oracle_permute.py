"""Pins of the token-permute oracle (HALOps "GEMM" page,
prefill_permute_to_masked_gemm section) against a hand-worked example,
closed forms and invariants that do not reuse the oracle's own steps."""
import os

import numpy as np

from oracle import permute as P

GOLD = os.path.join(os.path.dirname(__file__), "golden", "permute_small.txt")


def _golden():
    rec = {}
    for line in open(GOLD):
        if line.startswith("#") or not line.strip():
            continue
        key, *vals = line.split()
        rec[key] = vals
    return rec


def test_hand_worked_example():
    g = _golden()
    ids = np.array([int(v) for v in g["topk_ids"]], np.int64).reshape(4, 2)
    words = np.array([int(v, 16) for v in g["scale_words"]], np.uint32).view(np.int32).reshape(4, 1)
    x = np.arange(4 * 32, dtype=np.uint8).reshape(4, 32)     # row t holds bytes 32t .. 32t+31
    r = P.permute_to_masked(x, words, ids, 3, 128, 512, P.BROADCAST)
    assert r["map"].ravel().tolist() == [int(v) for v in g["map"]]
    assert r["counts"].tolist() == [int(v) for v in g["counts"]]
    for e, p, t in [(0, 0, 0), (2, 0, 0), (2, 1, 1), (1, 0, 2), (0, 1, 2), (0, 2, 3)]:
        assert np.array_equal(r["x"][e * 128 + p], x[t])
    assert int(r["written"].sum()) == 6
    assert r["scale"][0, 0].tolist() == [int(v, 16) for v in g["scale_token0"]]
    assert r["scale"][1, 0].tolist() == [int(v, 16) for v in g["scale_token2"]]


def test_overflowing_expert_keeps_the_first_rows():
    """200 tokens on one expert with max_token_num 128: rows 0..127 are the
    first 128 tokens in order, the rest are dropped (map -1)."""
    T, H = 200, 128
    x = np.random.default_rng(1).integers(0, 256, (T, 64), dtype=np.uint8)
    ids = np.zeros((T, 1), np.int64)
    sc = np.full((T, 1), 0x7F7F7F7F, np.int32)
    r = P.permute_to_masked(x, sc, ids, 2, 128, H, P.BROADCAST)
    assert r["counts"].tolist() == [128, 0]
    assert r["map"][:128, 0].tolist() == list(range(128))
    assert np.all(r["map"][128:, 0] == -1)
    assert np.array_equal(r["x"][:128], x[:128])
    assert not r["written"][128:].any()


def test_random_invariants_broadcast_and_direct():
    rng = np.random.default_rng(5)
    T, topk, E, M, H = 300, 4, 7, 256, 1024
    ids = rng.integers(-1, E + 2, (T, topk)).astype(np.int64)   # includes -1 and ids >= E
    x = rng.integers(0, 256, (T, 2 * H), dtype=np.uint8)
    words = rng.integers(0, 2 ** 32, (T, H // 512), dtype=np.uint64).astype(np.uint32).view(np.int32)
    direct = rng.integers(0, 256, (T, H // 32), dtype=np.uint8)
    # per-32 scales two other ways: the little-endian byte view of the words,
    # each byte repeated 4 times; and the direct bytes themselves
    want_b = np.repeat(words.view(np.uint8).reshape(T, H // 128), 4, axis=1)
    for mode, sc, want_sf in [(P.BROADCAST, words, want_b), (P.DIRECT, direct, direct)]:
        r = P.permute_to_masked(x, sc, ids, E, M, H, mode)
        valid = (ids >= 0) & (ids < E)
        assert np.array_equal(r["counts"], np.minimum(np.bincount(ids[valid], minlength=E), M))
        assert np.array_equal(r["map"] >= 0, valid)            # no expert overflows here
        for e in range(E):
            rows = np.sort(r["map"][ids == e])
            assert rows.tolist() == list(range(r["counts"][e])), "rows of an expert are 0..count-1"
        for t, j in zip(*np.nonzero(valid)):
            e, p = ids[t, j], r["map"][t, j]
            assert np.array_equal(r["x"][e * M + p], x[t])
            assert np.array_equal(r["scale"][e, p], want_sf[t])
        assert int(r["written"].sum()) == int(valid.sum())


def test_no_tokens():
    r = P.permute_to_masked(np.zeros((0, 16), np.uint8), np.zeros((0, 1), np.int32),
                            np.zeros((0, 8), np.int64), 4, 128, 512, P.BROADCAST)
    assert r["counts"].tolist() == [0, 0, 0, 0] and r["map"].shape == (0, 8)
