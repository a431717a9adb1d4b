"""Pins of the oracle's block copies of the split caches (swap_blocks,
copy_blocks): a hand-written 3-block example, untouched blocks, and the
reading that one table serves the K and V planes of every layer alike."""
import numpy as np

from oracle import rpa_oracle as O


def test_swap_blocks_hand_example():
    src = np.arange(3 * 2, dtype=np.uint16).reshape(3, 2)     # blocks [0 1] [2 3] [4 5]
    dst = np.full((4, 2), 9, dtype=np.uint16)
    out = O.swap_blocks(src, dst, np.array([[2, 0], [0, 3]]))
    np.testing.assert_array_equal(out, [[4, 5], [9, 9], [9, 9], [0, 1]])
    np.testing.assert_array_equal(dst, np.full((4, 2), 9))      # input left alone


def test_copy_blocks_every_layer_same_pairs():
    rng = np.random.default_rng(0)
    layers = [rng.integers(0, 255, (6, 4, 3), dtype=np.uint8) for _ in range(3)]
    out = O.copy_blocks(layers, np.array([[1, 4], [5, 0]]))
    for before, after in zip(layers, out):
        np.testing.assert_array_equal(after[4], before[1])
        np.testing.assert_array_equal(after[0], before[5])
        for b in (1, 2, 3, 5):
            np.testing.assert_array_equal(after[b], before[b])


def test_empty_table_is_identity():
    c = np.ones((2, 8), dtype=np.float32)
    np.testing.assert_array_equal(O.swap_blocks(c * 2, c, np.zeros((0, 2), np.int64)), c)
    np.testing.assert_array_equal(O.copy_blocks([c], np.zeros((0, 2), np.int64))[0], c)
