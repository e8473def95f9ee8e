"""Reference for dedicated ownership: which rank owns which matrix, and where
each owned matrix sits in the owner's packed buffer.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

DMuon landing page, intro: each matrix parameter is assigned to a single owner
rank.  Same page, "MoE": a balanced partition keeps any one rank from becoming
a straggler.  The pages do not give the balancing rule; the plain reading
taken here is the longest-processing-time greedy rule with the element count
as the cost:

  * visit matrices by element count, largest first; equal counts keep model
    order (a stable sort);
  * give each one to the owner with the smallest load so far; equal loads go
    to the lowest rank id.

Pack offsets: an owner's matrices are laid out in model order; each one starts
at the end of the previous one rounded up to a multiple of ``align`` elements.
"""

from __future__ import annotations


def partition_lpt(numels, n_owners: int):
    """Returns ``(owner_of_matrix, load_of_owner)``."""
    if n_owners <= 0:
        raise ValueError("n_owners must be positive")
    order = sorted(range(len(numels)), key=lambda i: -int(numels[i]))
    loads = [0] * n_owners
    owner = [-1] * len(numels)
    for i in order:
        best = 0
        for r in range(1, n_owners):
            if loads[r] < loads[best]:
                best = r
        owner[i] = best
        loads[best] += int(numels[i])
    return owner, loads


def round_up(x: int, align: int) -> int:
    return (x + align - 1) // align * align


def pack_offsets(numels, align: int):
    """Offsets of consecutive matrices in one buffer, each aligned to
    ``align`` elements.  Returns ``(offsets, total)`` where ``total`` is the
    end of the last matrix rounded up to ``align``."""
    offsets = []
    end = 0
    for n in numels:
        start = round_up(end, align)
        offsets.append(start)
        end = start + int(n)
    return offsets, round_up(end, align)
