"""Host-side bookkeeping of the Python layer against independent definitions
(CPU only): the candidate tile-pair count the module sizes its G_S slots
from, against the oracle's candidate definition (causal rule, sliding window,
64-row query tiles); the slot budget; and the per-slot byte count against the
C ABI's own workspace size query."""
import pytest

from oracle import backlite_oracle as orc


@pytest.fixture(scope="module")
def lib():
    from block_sparse_attention_fa_amd import _lib
    import os
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libbacklite.so is not built (run __graft_entry__.build())")
    return _lib


@pytest.mark.parametrize("n", [1, 64, 127, 128, 129, 300, 1000, 1536])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 1), (True, 100), (True, 200), (True, 5000)])
@pytest.mark.parametrize("q_tile", [64, 128])
def test_candidate_pairs_match_oracle(lib, n, causal, window, q_tile):
    """Candidate pairs per (batch, head): the oracle's candidate bitmap (a pair
    is a candidate iff some (row, key) of it is visible) summed."""
    cand = orc.candidates(n, causal, window=window, q_tile=q_tile)
    assert lib.candidate_pairs(n, causal, window, q_tile) == int(cand.sum())


@pytest.mark.parametrize("q_tile", [64, 128])
def test_slot_budget_and_slot_bytes(lib, q_tile):
    """Slots for a byte budget never exceed the candidate pairs, and one more
    slot adds exactly slot_bytes(q_tile) to the ABI's workspace size."""
    B, H, Hk, n, d = 1, 4, 2, 1000, 128
    pairs = B * H * lib.candidate_pairs(n, True, 0, q_tile)
    sb = lib.slot_bytes(q_tile)
    assert sb == q_tile * 128 * 2 + 4 * q_tile * 4
    assert lib.gs_slots_for_budget(B, H, n, True, 0, 10 * sb + sb // 2, None, q_tile) == 10
    assert lib.gs_slots_for_budget(B, H, n, True, 0, 10 ** 12, None, q_tile) == pairs
    assert lib.gs_slots_for_budget(B, H, n, True, 0, 0, None, q_tile) == 0
    w1 = lib.bwd_workspace_bytes_stored(B, H, Hk, n, d, 7, q_tile)
    w2 = lib.bwd_workspace_bytes_stored(B, H, Hk, n, d, 8, q_tile)
    assert w2 - w1 == sb
    assert lib.bwd_workspace_bytes_stored(B, H, Hk, n, d, 0, q_tile) == lib.bwd_workspace_bytes(B, H, Hk, n, d)
