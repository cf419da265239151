"""Pins of the plain-Python bucketing rules against hand-derived plans.

The expected lists below are worked out by hand from the rules stated on the
pages (HyperParallel-FSDP §6.6 / Figure 10; HyperParallel RFC item 3), not by
running the planner.
"""
import pytest

from oracle import plan_oracle as PO


def summary(batches):
    return [(b.M, b.N, b.count, b.transposed,
             [(s.param_index, s.first_matrix, s.num_matrices, s.elem_offset) for s in b.segments])
            for b in batches]


def test_core_shape_group():
    # [A,B], [A,1,B], [N,A,B] share the core shape (A,B) and fuse into one batch
    shapes = [(4, 6), (4, 1, 6), (3, 4, 6)]
    assert summary(PO.plan(shapes)) == [
        (4, 6, 5, False, [(0, 0, 1, 0), (1, 0, 1, 24), (2, 0, 3, 48)])]


def test_descending_and_stable_ties():
    # sizes: (2,3)x2 = 12 elems; (5,2)x1 = 10 (tall); (3,2)x2 = 12 -> tie keeps first-seen order
    shapes = [(2, 3), (5, 2), (2, 3), (3, 2), (2, 3, 2)]
    got = summary(PO.plan(shapes))
    # buckets: (2,3): params 0,2 -> 2 mats; (5,2): param 1; (3,2): param 3 (1 mat) + param 4 (2 mats)
    assert got == [
        (3, 2, 3, True, [(3, 0, 1, 0), (4, 0, 2, 6)]),
        (2, 3, 2, False, [(0, 0, 1, 0), (2, 0, 1, 6)]),
        (5, 2, 1, True, [(1, 0, 1, 0)]),
    ]
    # order=1 keeps creation order
    assert [b[:3] for b in summary(PO.plan(shapes, order=1))] == [(2, 3, 2), (5, 2, 1), (3, 2, 3)]


def test_cap_split_balanced():
    # cap 50 elements, matrices of 12 -> at most 4 per chunk; 10 matrices need 3 chunks -> 4 + 3 + 3
    got = summary(PO.plan([(10, 3, 4)], cap=50))
    assert [(b[2], b[4]) for b in got] == [
        (4, [(0, 0, 4, 0)]), (3, [(0, 4, 3, 0)]), (3, [(0, 7, 3, 0)])]
    # 8 matrices -> 4 + 4 (no smaller chunk when the count divides)
    assert [b[2] for b in summary(PO.plan([(8, 3, 4)], cap=50))] == [4, 4]
    # one matrix above the cap still runs whole
    assert summary(PO.plan([(8, 8)], cap=10)) == [(8, 8, 1, False, [(0, 0, 1, 0)])]


def test_square_not_transposed():
    assert PO.plan([(7, 7)])[0].transposed is False
    assert PO.plan([(8, 7)])[0].transposed is True
    assert PO.plan([(7, 8)])[0].transposed is False


def test_decoder_workload_plan():
    # 32 layers x (q,k,v,o 4096^2; gate, up 11008x4096; down 4096x11008), cap 2^29
    shapes = []
    for _ in range(32):
        shapes += [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
    b = PO.plan(shapes)
    # 2^29 // 4096^2 = 32; 2^29 // (11008*4096) = 11, so 64 matrices -> 6 chunks (11,11,11,11,10,10)
    # and 32 -> 3 chunks (11,11,10); larger batches first, ties in creation order
    counts = [(x.M, x.N, x.count) for x in b]
    assert counts == ([(4096, 4096, 32)] * 4 + [(11008, 4096, 11)] * 4 + [(4096, 11008, 11)] * 2
                      + [(11008, 4096, 10)] * 2 + [(4096, 11008, 10)])
    assert sum(x.count for x in b if x.M == 11008) == 64


def test_moe_and_large_plans():
    b = PO.plan([(32, 24, 10240), (64, 2048, 7168)])
    # 2^29 // (2048*7168) = 36, so 64 experts take 2 chunks of 32
    assert [(x.M, x.N, x.count) for x in b] == [(2048, 7168, 32), (2048, 7168, 32), (24, 10240, 32)]
    shapes = [(8192, 28672)] * 16 + [(28672, 8192)] * 16
    b = PO.plan(shapes)
    assert len(b) == 16 and all(x.count == 2 for x in b)
    assert [x.transposed for x in b] == [False] * 8 + [True] * 8


@pytest.mark.parametrize("bad", [(5,), (2, 3, 4, 5), (0, 4), (3, 0, 2)])
def test_rejects(bad):
    with pytest.raises(ValueError):
        PO.plan([bad])
