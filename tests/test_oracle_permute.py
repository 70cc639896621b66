"""Pins of the oracle's permutation (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle.moe import permute, topk_softmax

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _routing(T, E, k, seed):
    l = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    return topk_softmax(l, k)[0]


def _bucket_brute(idx, E):
    """Expert-major buckets by walking experts, then tokens, then slots."""
    T, k = idx.shape
    rows = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    rows.append((t, j))
    return rows


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (100, 16, 4), (37, 64, 10), (1, 5, 5), (300, 512, 10)])
def test_permute_matches_bucket_walk(T, E, k):
    idx = _routing(T, E, k, seed=T + E + k)
    counts, offsets, row_token, row_of_slot = permute(idx, E)
    rows = _bucket_brute(idx, E)
    assert row_token.tolist() == [t for t, _ in rows]
    for r, (t, j) in enumerate(rows):
        assert row_of_slot[t * k + j] == r
    assert counts.tolist() == [int((idx == e).sum()) for e in range(E)]


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (513, 40, 7)])
def test_permute_invariants_and_round_trip(T, E, k):
    idx = _routing(T, E, k, seed=9)
    counts, offsets, row_token, row_of_slot = permute(idx, E)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    for e in range(E):
        grp = row_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(grp) > 0)            # ascending, no repeats
        assert np.all(np.any(idx[grp] == e, axis=1))
    assert sorted(row_of_slot.tolist()) == list(range(T * k))
    # gather then inverse gather is the identity, bit for bit
    x = np.random.default_rng(1).standard_normal((T, 24)).astype(np.float32)
    x_perm = x[row_token]
    for j in range(k):
        assert np.array_equal(x_perm[row_of_slot.reshape(T, k)[:, j]], x)


def test_permuted_buffer_rows_of_the_qwen_prefill():
    """The pages' permuted buffer for the 8192-token top-10 prefill has 81920
    rows (golden fixture); the oracle's row space has T*k rows."""
    g = json.load(open(os.path.join(GOLDEN, "permuted_buffer_shape.json")))
    T, k = g["tokens"], g["top_k"]
    idx = np.stack([np.random.default_rng(0).permutation(512)[:k] for _ in range(4)])
    idx = np.tile(idx, (T // 4, 1))
    counts, offsets, row_token, row_of_slot = permute(idx, 512)
    assert row_token.shape[0] == g["rows"] == offsets[-1]


def test_empty_experts_and_single_expert():
    idx = np.zeros((10, 1), np.int32) + 3
    counts, offsets, row_token, row_of_slot = permute(idx, 6)
    assert counts.tolist() == [0, 0, 0, 10, 0, 0]
    assert offsets.tolist() == [0, 0, 0, 0, 10, 10, 10]
    assert row_token.tolist() == list(range(10))
    assert row_of_slot.tolist() == list(range(10))
