"""Pins for the oracle state hash (CPU only).

OPEN-1B paper, Appendix B (a sharded canonical per-step state hash) and the
legend of Figure 11 (the hash is BLAKE2b); section 3.2 "Optimizer-state
precision" (state hashed in FP32).  The function is BLAKE2b of RFC 7693 in
the tree mode of the BLAKE2 paper (section 2.10), with leaf 4096 bytes,
fanout 16, depth 255, inner digests and output 32 bytes, personalisation
"repro_state_v1", over the little-endian bytes of [w | m | v].

Python's hashlib implements BLAKE2b with the same tree parameters
independently of this repository, so it pins both the compression function
and the framing.
"""
import hashlib
import os

import numpy as np
import pytest

import oracle

PERSON = b"repro_state_v1"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "blake2b_rfc7693.txt")


def _node(data, offset, depth, last):
    return hashlib.blake2b(data, digest_size=32, fanout=16, depth=255, leaf_size=4096,
                           node_offset=offset, node_depth=depth, inner_size=32, last_node=last,
                           person=PERSON).digest()


def _hashlib_tree(words):
    b = np.asarray(words, np.float32).astype("<f4").tobytes()
    L = max(1, -(-len(b) // 4096))
    level = [_node(b[i * 4096:(i + 1) * 4096], i, 0, i == L - 1) for i in range(L)]
    depth = 1
    while True:
        parents = -(-len(level) // 16)
        level = [_node(b"".join(level[j * 16:(j + 1) * 16]), j, depth, j == parents - 1)
                 for j in range(parents)]
        depth += 1
        if len(level) == 1:
            return level[0]


def test_rfc7693_known_answer():
    with open(GOLDEN) as fh:
        rows = [ln.split() for ln in fh if ln.strip() and not ln.startswith("#")]
    for msg, hexdigest in rows:
        assert oracle.blake2b(msg.encode(), 64).hex() == hexdigest


def test_sequential_mode_matches_hashlib():
    rng = np.random.default_rng(0)
    for n in (0, 1, 127, 128, 129, 255, 256, 1000, 4096, 4097):
        data = rng.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert oracle.blake2b(data, 64) == hashlib.blake2b(data).digest()
        assert oracle.blake2b(data, 32, PERSON) == hashlib.blake2b(data, digest_size=32, person=PERSON).digest()


# Word counts: empty; one word; a partial leaf; exactly one leaf; one leaf and
# a word; 16 leaves (one level above the leaves); 17 leaves (two levels);
# 33 leaves; 16*16 leaves + 5 words (three levels); 5000 leaves (four).
@pytest.mark.parametrize("n", [0, 1, 1023, 1024, 1025, 16 * 1024, 16 * 1024 + 1, 33 * 1024,
                               16 * 16 * 1024 + 5, 5000 * 1024])
def test_tree_mode_matches_hashlib(n):
    w = np.random.default_rng(n).standard_normal(n).astype(np.float32)
    assert oracle.state_hash(w) == _hashlib_tree(w)


def test_leaf_digests_match_hashlib():
    w = np.random.default_rng(9).standard_normal(5 * 1024 + 7).astype(np.float32)
    b = w.astype("<f4").tobytes()
    leaves = oracle.state_hash_leaves(w, 2, 4)
    for i in range(4):
        leaf = 2 + i
        assert leaves[i].tobytes() == _node(b[leaf * 4096:(leaf + 1) * 4096], leaf, 0, leaf == 5)


def test_one_leaf_entry_matches_the_leaf_level():
    w = np.random.default_rng(10).standard_normal(7 * 1024 + 100).astype(np.float32)
    leaves = oracle.state_hash_leaves(w, 0, 8)
    for i in range(8):
        assert oracle.state_hash_one_leaf(w[i * 1024:(i + 1) * 1024], i, i == 7) == leaves[i].tobytes()


def test_single_changes_move_the_digest():
    w = np.random.default_rng(1).standard_normal(3 * 65536).astype(np.float32)
    d0 = oracle.state_hash(w)
    w1 = w.copy()
    w1.view(np.uint32)[123_457] ^= 1  # one bit of one word
    assert oracle.state_hash(w1) != d0
    w2 = w.copy()
    w2[[10, 11]] = w2[[11, 10]]  # swap two words
    assert oracle.state_hash(w2) != d0
    # -0.0 and +0.0 hash differently: the hash sees words, not values.
    z = np.zeros(4, np.float32)
    assert oracle.state_hash(z) != oracle.state_hash(-z)
