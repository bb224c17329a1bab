"""Ring pointer state machine (CPU only): invariants under random operation sequences."""
import hypothesis.strategies as st
from hypothesis import given, settings

from oracle.ring import Ring


ops = st.lists(st.tuples(st.sampled_from(["decode", "spec", "flush", "flush_all"]),
                         st.integers(0, 8)), max_size=60)


@settings(max_examples=300, deadline=None)
@given(L=st.integers(1, 8), smax=st.integers(1, 8), seq=ops)
def test_ring_invariants(L, smax, seq):
    smax = min(smax, L)
    cap = L + smax - 1
    r = Ring(cap=cap, L=L)
    folded = []  # token indices folded, in order
    for op, arg in seq:
        if op == "decode":
            if r.count + 1 > cap:
                continue
            slot = r.decode()
            assert slot == (r.start + r.count - 1) % cap
            r.flush_if_full()
        elif op == "spec":
            S = 1 + arg % smax
            if r.count + S > cap:
                continue
            before = (r.start, r.count, r.position, r.committed)
            slots = r.spec_append(S)
            assert len(set(slots)) == S
            committed_slots = set(r.slots())
            assert not committed_slots & set(slots)  # drafts never overwrite committed entries
            a = arg % (S + 1)
            r.rollback(a)
            if a == 0:
                assert (r.start, r.count, r.position, r.committed) == before
            r.flush_if_full()
        elif op == "flush":
            r.flush_if_full()
        else:
            r.flush_all()
        assert 0 <= r.count <= cap
        assert r.count < L or r.count <= cap
        assert r.position + r.count == r.committed
        assert len(set(r.slots())) == r.count
    # each flush folds a contiguous run starting at the previous checkpoint position
    pos = 0
    for p0, n in r.flushes:
        assert p0 == pos and n >= 1
        pos += n
    assert pos == r.position


def test_flush_folds_exactly_L_and_keeps_remainder():
    r = Ring(cap=7, L=4)
    r.spec_append(4)
    r.rollback(4)
    r.flush_if_full()
    assert (r.position, r.count) == (4, 0)
    for _ in range(3):
        r.decode()
    r.spec_append(4)
    r.rollback(4)  # count 7 == cap
    assert r.count == 7
    assert r.flush_if_full()
    assert (r.position, r.count, r.start) == (8, 3, 1)
