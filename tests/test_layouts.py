"""Host-side layouts of the fp8 pools the union kernel reads (no GPU): each
(page, KV head) tile is stored in the MFMA operand order the kernel's lanes
load, 64 lanes x 16 bytes per block.  Checked against the operand layout
of v_mfma_f32_32x32x64 as the kernel uses it: lane l holds row l % 32 and
the half l // 32 of each 64-wide k block."""
import numpy as np
import pytest

from query_aware_sparse_amd.staging import mfma_token_order, union_k_order, union_v_order


@pytest.mark.parametrize("S", [32, 64])
def test_orders_are_permutations(S):
    for order in (union_k_order(S), union_v_order(S)):
        assert np.array_equal(np.sort(order), np.arange(S * 128))
    assert np.array_equal(np.sort(mfma_token_order(S)), np.arange(S))


def test_k_block_holds_the_lane_operand_bytes():
    # S = 64: block (tau=1, ks=0, c=1) is the 6th (index 5); lane 33 is row 1,
    # half 1, so its bytes are token 33, dims 32 + 16 .. 32 + 31
    order = union_k_order(64)
    j = (5 * 64 + 33) * 16
    assert order[j:j + 16].tolist() == [33 * 128 + 48 + b for b in range(16)]
    # every 16-byte piece is one token row's consecutive dims
    pieces = order.reshape(-1, 16)
    assert np.all(np.diff(pieces, axis=1) == 1)


def test_v_block_holds_the_lane_operand_bytes():
    # S = 64: block (dt=2, c=1) is index 5; lane 40 is dim 72, half 1, so its
    # k slots are 32 + 16 + [0, 16).  Slot 48 holds token 36 (w = 4: odd
    # quad, tau = 1, first of its quad), slot 49 token 37.
    order = union_v_order(64)
    j = (5 * 64 + 40) * 16
    assert order[j] == 36 * 128 + 72 and order[j + 1] == 37 * 128 + 72
    # every byte of a piece is the same dim, and the 16 tokens are those of
    # the lane's k slots
    tok = mfma_token_order(64)
    for lane in (0, 17, 40, 63):
        for dt in range(4):
            for c in range(2):
                j = ((dt * 2 + c) * 64 + lane) * 16
                dim = 32 * dt + lane % 32
                slots = 32 * (lane // 32) + 16 * c + np.arange(16)
                assert order[j:j + 16].tolist() == (tok[slots] * 128 + dim).tolist()


def test_token_order_matches_the_pv_k_slots():
    # the P bytes a lane holds for k slots 0..31 of a 32-token block come from
    # the QK result rows 8 (e/4) + 4 hf + e%4: both halves' slots together
    # cover the block once, in that order
    tok = mfma_token_order(32)
    for hf in range(2):
        got = tok[16 * hf:16 * hf + 16].tolist()
        assert got == [8 * (e // 4) + 4 * hf + e % 4 for e in range(16)]
