"""Pins for tests/rescale_rule.py, the CPU replay of the kernels' lazy-rescale
rule that the GPU tests use to prove their workloads reach the rescale branch."""

import numpy as np

from mla_paged_kv_amd import workloads as W
from tests import rescale_rule as RR


def test_count_moves_hand_built():
    # one row, 4 tiles of 32 keys; tile maxima 0, 7.9, 20, 27 (log2 units):
    # 7.9 stays below 0 + 8, 20 moves the reference (0 -> 20), 27 does not (< 28)
    s = np.full((1, 128), -50.0)
    s[0, 5], s[0, 40], s[0, 70], s[0, 100] = 0.0, 7.9, 20.0, 27.0
    moves, amb = RR.count_moves(s, 0, 128, margin=0.5)
    assert (moves, amb) == (1, 1)  # 7.9 is within 0.5 of the threshold
    # a piece starting at key 64 begins afresh: its first tile (max 20) is not a move
    assert RR.count_moves(s, 64, 128)[0] == 0
    # masked keys (-inf) never move the reference
    s2 = np.full((2, 64), -np.inf)
    s2[0, :32] = 1.0
    assert RR.count_moves(s2, 0, 64) == (0, 0)


def test_pieces_follow_the_partition():
    # [1, 700, 2049] in 5 parts: 1 + 11 + 33 = 45 blocks, 9 blocks per part
    got = RR.pieces([1, 700, 2049], 5)
    assert got == [(0, 0, 1), (1, 0, 512), (1, 512, 700), (2, 0, 384), (2, 384, 960), (2, 960, 1536),
                   (2, 1536, 2049)]


def test_plain_inputs_never_move_but_planted_ones_do():
    w = W.dense_workload("plain", 1, 3, 1, 128, [1, 700, 2049], pool_pages=60)
    assert RR.moves_for(w, 5)[0] == 0
    w = W.dense_workload("planted", 1, 3, 1, 128, [1, 700, 2049], pool_pages=60)
    W.plant_dense(w, [(1, 150, 15.0), (2, 2048, 50.0)])
    assert RR.moves_for(w, 5)[0] == 2 * 128
