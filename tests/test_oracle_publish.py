"""Pins of the oracle's zero-copy publish (mailbox stand-in).

What the pages fix: the unpooler page's module description (zero-copy
epilogue: the GEMM also writes its output into the slot this rank owns in
the following boundary's mailbox, at the publish stage, with negative zero
replaced by positive zero, and then sets the active-stage word; with a
ticket, the ticket word's high half selects the stage and the call leaves
the stage word alone) and the pooler_gather page (a mailbox holds BF16
[3, tp, capacity, hidden / tp]; negative zero marks an entry not yet
written).  The checks below are
a hand-worked case and properties that hold for any input, not a second copy
of the oracle's loop.
"""
import numpy as np
import pytest

import oracle

POISON = 0x1234


def _mailbox(tp, capacity, width):
    return np.full((3, tp, capacity, width), POISON, dtype=np.uint16)


def test_publish_worked_case():
    # tp 2, rank 1, capacity 3, width 4, two rows, stage 2.
    y = np.array([[0x8000, 0x0000, 0x3F80, 0xBF80],     # -0, +0, 1, -1
                  [0x8001, 0x7F80, 0xFFC0, 0x0001]],    # -tiny, inf, NaN, +tiny
                 dtype=np.uint16)
    mb = _mailbox(2, 3, 4)
    st = np.array([2, 0], dtype=np.int32)
    assert oracle.mailbox_publish(y, mb, 1, stage_state=st) == 2
    want = np.array([[0x0000, 0x0000, 0x3F80, 0xBF80],  # only -0 changes
                     [0x8001, 0x7F80, 0xFFC0, 0x0001]], dtype=np.uint16)
    assert np.array_equal(mb[2, 1, :2], want)
    assert np.all(mb[2, 1, 2] == POISON)                  # row 2 >= M untouched
    other = mb.copy()
    other[2, 1, :2] = POISON
    assert np.all(other == POISON)                        # no other slot touched
    assert st.tolist() == [2, 2]                          # the active stage is set


def test_publish_ticket_stage_uses_upper_half_and_stores_no_word():
    y = np.array([[0x8000, 0x4000]], dtype=np.uint16)
    mb = _mailbox(1, 1, 2)
    ticket = np.array([(1 << 16) | 0x0005], dtype=np.int32)
    st = np.array([2, 0], dtype=np.int32)  # present but not used with a ticket
    assert oracle.mailbox_publish(y, mb, 0, stage_state=st, ticket=ticket) == 1
    assert mb[1, 0, 0].tolist() == [0x0000, 0x4000]
    assert np.all(mb[0] == POISON) and np.all(mb[2] == POISON)
    assert ticket.tolist() == [(1 << 16) | 5] and st.tolist() == [2, 0]


@pytest.mark.parametrize("stage_state,ticket", [([3, 7], None), ([-1, 7], None),
                                                (None, [3 << 16]), (None, [0x7FFF0000])])
def test_publish_outside_stages_writes_nothing(stage_state, ticket):
    y = np.zeros((1, 8), dtype=np.uint16)
    mb = _mailbox(2, 1, 8)
    st = None if stage_state is None else np.array(stage_state, dtype=np.int32)
    tk = None if ticket is None else np.array(ticket, dtype=np.int32)
    assert oracle.mailbox_publish(y, mb, 1, stage_state=st, ticket=tk) == -1
    assert np.all(mb == POISON)
    if st is not None:
        assert st.tolist() == stage_state


@pytest.mark.parametrize("seed", range(6))
def test_publish_properties(seed):
    rng = np.random.default_rng(seed)
    tp, capacity, width = int(rng.integers(1, 5)), int(rng.integers(1, 17)), 16 * int(rng.integers(1, 9))
    M = int(rng.integers(1, capacity + 1))
    rank = int(rng.integers(0, tp))
    stage = int(rng.integers(0, 3))
    y = rng.integers(0, 1 << 16, size=(M, width), dtype=np.uint16)
    y[rng.random((M, width)) < 0.2] = 0x8000
    y[rng.random((M, width)) < 0.1] = 0x0000
    mb = _mailbox(tp, capacity, width)
    st = np.array([stage, -5], dtype=np.int32)
    assert oracle.mailbox_publish(y, mb, rank, stage_state=st) == stage
    slot = mb[stage, rank, :M]
    # numerically the same values (NaN where y is NaN), and never the sentinel
    yv, sv = oracle.bf16_value(y), oracle.bf16_value(slot)
    assert np.array_equal(np.isnan(yv), np.isnan(sv))
    assert np.all((yv == sv) | np.isnan(yv))
    assert not np.any(slot == 0x8000)
    # every non-zero pattern is copied bit for bit; zeros come out as +0
    nz = (y & 0x7FFF) != 0
    assert np.array_equal(slot[nz], y[nz]) and np.all(slot[~nz] == 0)
    rest = mb.copy()
    rest[stage, rank, :M] = POISON
    assert np.all(rest == POISON)
    assert st.tolist() == [stage, stage]
