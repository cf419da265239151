"""Plain-Python statement of the host-side shape bucketing (the batch plan).

TEST INFRASTRUCTURE ONLY (same rules as ``muon_oracle``): the C++ planner in
the library is compared with this, entry by entry.

Rules, from HyperParallel-FSDP §6.6 / Figure 10(a) and HyperParallel RFC
item 3:

* [A,B], [A,1,B] and [N,A,B] share the core shape (A,B): the first two are one
  matrix, the third is N matrices (HyperParallel-FSDP §6.3: an expert tensor is
  E independent matrices).  Any 3-D shape whose middle dimension is 1 is read
  as [A,1,B].
* Matrices of one core shape are concatenated along a batch axis, parameter by
  parameter, in input order.
* A batch holds at most ``cap`` elements (the "memory-safe batching" cap of
  §6.6, read as 2^29 elements; one GPU, so the shard-group scaling is 1).  A
  chunk holds at most floor(cap / (A*B)) matrices (at least one, so a single
  matrix above the cap still runs whole).  The section fixes only the cap, so
  a bucket is cut into as few chunks as that allows, of sizes that differ by
  at most one, the larger ones first (64 matrices at 36 per chunk: 32 + 32,
  not 36 + 28).
* Batches run in descending size (Figure 10(b), Algorithm 2); equal sizes keep
  their creation order.
* A batch whose matrices have more rows than columns is marked transposed
  (the transpose-first rule of §6.6; square matrices are not).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Sequence, Tuple

DEFAULT_CAP = 1 << 29


@dataclass
class Segment:
    param_index: int
    first_matrix: int
    num_matrices: int
    elem_offset: int


@dataclass
class Batch:
    M: int
    N: int
    count: int
    transposed: bool
    segments: List[Segment]

    @property
    def elems(self) -> int:
        return self.count * self.M * self.N


def core_shape(shape: Sequence[int]) -> Tuple[int, int, int]:
    """(matrices, M, N) of a parameter shape, or ValueError."""
    if len(shape) == 2:
        n_mat, M, N = 1, shape[0], shape[1]
    elif len(shape) == 3 and shape[1] == 1:
        n_mat, M, N = 1, shape[0], shape[2]
    elif len(shape) == 3:
        n_mat, M, N = shape
    else:
        raise ValueError("only 2-D and 3-D parameters are Muon matrices")
    if min(shape) <= 0:
        raise ValueError("zero-size dimension")
    return n_mat, M, N


def plan(shapes: Sequence[Sequence[int]], cap: int = DEFAULT_CAP, order: int = 0) -> List[Batch]:
    buckets = {}          # (M,N) -> list of (param_index, matrix_index); dict keeps first-seen order
    for pi, s in enumerate(shapes):
        n_mat, M, N = core_shape(s)
        buckets.setdefault((M, N), []).extend((pi, mi) for mi in range(n_mat))
    batches: List[Batch] = []
    for (M, N), mats in buckets.items():
        per = M * N
        max_count = max(1, cap // per)
        n_chunks = -(-len(mats) // max_count)
        sizes = [len(mats) // n_chunks + (1 if c < len(mats) % n_chunks else 0) for c in range(n_chunks)]
        starts = [sum(sizes[:c]) for c in range(n_chunks)]
        for start, size in zip(starts, sizes):
            chunk = mats[start:start + size]
            segs: List[Segment] = []
            for k, (pi, mi) in enumerate(chunk):
                if segs and segs[-1].param_index == pi and segs[-1].first_matrix + segs[-1].num_matrices == mi:
                    segs[-1].num_matrices += 1
                else:
                    segs.append(Segment(pi, mi, 1, k * per))
            batches.append(Batch(M, N, len(chunk), M > N, segs))
    if order == 0:
        batches = sorted(batches, key=lambda b: -b.elems)   # sorted() is stable
    return batches
