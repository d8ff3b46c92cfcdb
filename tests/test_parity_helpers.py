"""The GPU tests' error measures (tests/parity.py) on planted differences, on
the CPU: a whole-tensor norm can hide one wrong tile, the per-pair and
per-chunk measures must not."""
import numpy as np
import torch

import parity


def _pair():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((2, 2048, 4, 64))
    mine = torch.from_numpy(ref * (1 + 1e-3 * rng.standard_normal(ref.shape)))
    return ref, mine


def test_clean_tensor_passes_every_bound():
    ref, mine = _pair()
    e = parity.token_errors(mine, ref)
    assert e["total"] < 2e-3 and e["pair"].max() < 2e-3 and e["chunk_max"] < 3e-3
    parity.check("x", e, 2e-2)


def test_one_wrong_tile_fails_the_chunk_bound_only():
    ref, mine = _pair()
    mine[1, 128:144, 2, :16] = 0.0  # a 16 x 16 tile never written
    e = parity.token_errors(mine, ref)
    assert e["total"] < 2e-2           # hidden in the whole tensor
    assert e["chunk_at"] == (1, 2, 2)  # sequence 1, head 2, chunk 2
    assert e["chunk_max"] > 5e-2


def test_wrong_pair_is_located():
    ref, mine = _pair()
    mine[0, :, 3] *= 1.05
    e = parity.token_errors(mine, ref)
    assert np.unravel_index(int(np.argmax(e["pair"])), e["pair"].shape) == (0, 3)
    assert abs(e["pair"][0, 3] - 0.05) < 2e-3


def test_packed_sequences_and_empty_members():
    rng = np.random.default_rng(1)
    lens = (5, 0, 130, 64)
    cu = np.cumsum((0,) + lens)
    ref = rng.standard_normal((1, sum(lens), 2))
    mine = ref.copy()
    mine[0, cu[2] + 70, 1] += 1.0  # sequence 2, head 1, chunk 1
    e = parity.token_errors(torch.from_numpy(mine), ref, cu=list(cu))
    assert e["chunk_at"] == (2, 1, 1)
    assert e["pair"][1].max() == 0.0 and e["pair"][0].max() == 0.0


def test_state_errors_per_pair():
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((3, 2, 8, 8))
    mine = ref.copy()
    mine[2, 1] *= 1.1
    e = parity.state_errors(torch.from_numpy(mine), ref)
    assert abs(e["pair"][2, 1] - 0.1) < 1e-12 and e["pair"][0].max() == 0.0


def test_blocks_of_few_values_are_left_to_the_tensor_bound():
    # a per-token scalar: a one-token sequence, and a one-token tail chunk
    rng = np.random.default_rng(3)
    lens = (1, 65, 200)
    cu = np.cumsum((0,) + lens)
    ref = rng.standard_normal((1, sum(lens), 2))
    mine = ref.copy()
    mine[0, 0, 0] *= 1.5          # the one-token sequence
    mine[0, cu[1] + 64, 1] *= 1.5  # the tail chunk of sequence 1
    e = parity.token_errors(torch.from_numpy(mine), ref, cu=list(cu))
    assert e["pair"][0].max() == 0.0
    assert e["chunk_max"] == 0.0
    assert e["total"] > 0.0
    # the same one-token values with 64 values per token are checked
    ref4 = rng.standard_normal((1, sum(lens), 2, 64))
    mine4 = ref4.copy()
    mine4[0, cu[1] + 64, 1] *= 1.5
    e4 = parity.token_errors(torch.from_numpy(mine4), ref4, cu=list(cu))
    assert e4["chunk_at"] == (1, 1, 1) and e4["chunk_max"] > 0.4
