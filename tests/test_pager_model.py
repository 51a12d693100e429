"""The page-pool policy model (``oracle.pager``) on its own, against page ids,
events and statistics worked out by hand from the policy it states."""
from oracle.pager import PagerModel


def test_model_page_choices_derived_by_hand():
    """The policy model alone, against page ids and events worked out by hand
    from the stated policy (lowest empty page first, then the cached page
    released longest ago; pages released last to first)."""
    m = PagerModel(6, 4, 6)
    S, R = 0, 1
    assert m.add_sequence(1, list(range(12)))[1] == list(range(12))  # pages 0 1 2
    assert m.add_sequence(2, list(range(100, 108)))[1] == [12 + i for i in range(8)]  # 3 4
    assert m.drain_events() == [(S, 0), (S, 1), (S, 2), (S, 3), (S, 4)]
    assert m.free_sequence(1) == 0                      # released 2, then 1, then 0
    st, slots, cached = m.add_sequence(4, list(range(300, 308)))
    assert (st, cached) == (0, 0)
    assert [s // 4 for s in slots[::4]] == [5, 2]       # empty page 5, then evict 2
    assert m.drain_events() == [(R, 2), (S, 5), (S, 2)]
    assert m.add_sequence(5, list(range(8)))[1:] == (list(range(8)), 8)  # 0 1 reused
    assert m.free_sequence(2) == 0                      # released 4, then 3
    st, slots, cached = m.add_sequence(6, [1, 2, 3])
    assert [s // 4 for s in slots] == [4, 4, 4]         # no empty page: evict 4
    assert m.drain_events() == [(R, 4)]
    rows, lens = m.block_tables([4, 5, 6])
    assert rows == [[5, 2, -1, -1, -1, -1], [0, 1, -1, -1, -1, -1], [4, -1, -1, -1, -1, -1]]
    assert lens == [8, 8, 3]
    assert m.stats() == {"num_pages": 6, "in_use": 5, "cached_free": 1, "empty_free": 0,
                         "registered": 5, "live_sequences": 3, "prefix_hit_tokens": 8,
                         "evictions": 2, "cow_copies": 0}
    # fork, then the first append to the shared partial page moves it
    assert m.fork(6, 7) == 0
    st, slot, copy = m.append(7, 9)
    assert (st, copy) == (0, (4, 3)) and slot == 3 * 4 + 3   # page 3: the only free page
    st, slot, copy = m.append(6, 9)
    assert (st, copy, slot) == (0, None, 4 * 4 + 3)          # page 4 private again: in place
