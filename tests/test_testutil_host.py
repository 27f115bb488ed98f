"""The parity helpers themselves (CPU): the per-chunk ratio catches an error
confined to small-magnitude rows that the chain-wide ratio lets through."""
import numpy as np

from kda_testutil import chunk_rel_err, rel_err


def test_chunk_ratio_catches_small_rows():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((200, 128))
    ref[64:128] *= 1e-3             # a chunk after strong decay
    x = ref.copy()
    x[64:128] += 1e-4               # 10% of that chunk's magnitude
    assert rel_err(x, ref) < 1e-3   # invisible chain-wide
    e, c = chunk_rel_err(x, ref)
    assert c == 1 and 0.02 < e < 0.2


def test_chunk_ratio_ragged_tail_and_zero_chunk():
    ref = np.ones((130, 4))
    ref[64:128] = 0.0
    x = ref.copy()
    assert chunk_rel_err(x, ref) == (0.0, -1)
    x[129, 0] += 0.5                # the 2-row tail chunk
    e, c = chunk_rel_err(x, ref)
    assert c == 2 and abs(e - 0.5) < 1e-12
    x[100, 1] = 1e-9                # nonzero where the reference chunk is all zero
    e, c = chunk_rel_err(x, ref)
    assert c == 1 and e == np.inf
