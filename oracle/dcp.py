"""Reference of the Dynamic Context Parallelism schedule (plain Python).

TEST INFRASTRUCTURE ONLY, like ref.py: only the test suite and the benchmark's
CPU-baseline leg use it; it shares no code with the library and does not import it.

Constraints taken from the verl page "Dynamic Context Parallelism": every DP x CP
rank sees the same mini-batch; the scheduler packs under a per-rank token limit
(max_seqlen_per_dp_cp_rank: the static run's packed budget divided by its CP
size, 16384 / 4 = 4096 for static CP4); CP groups are power-of-two subgroups of
the DP x CP ranks plus the full group when needed (so a non-power-of-two world
leaves no rank out); the world size is an even integer of at least two.  The
"Megatron 6D parallelism guide" (section 6.1) adds that the CP size follows the
sequence lengths so that short sequences are not split.

The pages do not print the assignment rule.  The reading taken (the same one the
library documents):
  1. group sizes: 1, 2, 4, ... up to the world size, and the world size;
     sample i gets the smallest size g with ceil(L_i / g) <= limit;
  2. the sample is cut into g contiguous pieces of ceil(L_i / g) tokens (the last
     one what is left), piece r on rank first + r of its group;
  3. samples go in order of decreasing (g, L), ties by index, each to the first
     micro-batch that takes it: an existing group of size g whose ranks all stay
     within the limit, else a new group of size g at the lowest aligned start
     (a multiple of g; the full group starts at 0) whose ranks are in no group
     yet; failing both, a new micro-batch.

The pages print no worked schedule to compare with.  The tests pin this reference
instead with closed forms, hand-derived placements, invariants checked from the
constraints above, and the workload generator's per-sample CP rule.
"""
from __future__ import annotations

from typing import Dict, List


def group_sizes(world: int) -> List[int]:
    """Powers of two up to `world`, then `world` itself if it is not one."""
    out, g = [], 1
    while g <= world:
        out.append(g)
        g *= 2
    if out[-1] != world:
        out.append(world)
    return out


def cp_size_of(length: int, world: int, limit: int) -> int:
    for g in group_sizes(world):
        if -(-length // g) <= limit:
            return g
    raise ValueError(f"a sample of {length} tokens does not fit {world} ranks x {limit}")


def pieces(length: int, g: int) -> List[int]:
    """Tokens on each rank of a group of g ranks: ceil(L/g) each, the last the remainder."""
    p = -(-length // g)
    return [max(0, min(p, length - r * p)) for r in range(g)]


def dcp_schedule_ref(lengths, world: int, limit: int) -> Dict:
    if world < 2 or world % 2:
        raise ValueError("world must be an even integer >= 2")
    if limit < 1:
        raise ValueError("limit must be >= 1")
    n = len(lengths)
    lengths = [int(x) for x in lengths]
    if any(x < 0 for x in lengths):
        raise ValueError("negative length")
    cp = [cp_size_of(x, world, limit) for x in lengths]
    order = sorted(range(n), key=lambda i: (-cp[i], -lengths[i], i))

    batches = []   # each: {"load": [..world..], "groups": [[first, size, count], ...], "owned": set()}
    mb, first_rank, slot = [0] * n, [0] * n, [0] * n
    for i in order:
        g, share = cp[i], pieces(lengths[i], cp[i])
        placed = False
        for b, batch in enumerate(batches):
            for grp in batch["groups"]:
                first, size, _ = grp
                if size == g and all(batch["load"][first + r] + share[r] <= limit for r in range(g)):
                    for r in range(g):
                        batch["load"][first + r] += share[r]
                    mb[i], first_rank[i], slot[i] = b, first, grp[2]
                    grp[2] += 1
                    placed = True
                    break
            if placed:
                break
            starts = range(0, world - g + 1, g) if g & (g - 1) == 0 else [0]
            for first in starts:
                ranks = range(first, first + g)
                if any(r in batch["owned"] for r in ranks):
                    continue
                if any(batch["load"][first + r] + share[r] > limit for r in range(g)):
                    continue
                batch["owned"].update(ranks)
                batch["groups"].append([first, g, 1])
                for r in range(g):
                    batch["load"][first + r] += share[r]
                mb[i], first_rank[i], slot[i] = b, first, 0
                placed = True
                break
            if placed:
                break
        if not placed:
            batch = {"load": [0] * world, "groups": [[0, g, 1]], "owned": set(range(g))}
            for r in range(g):
                batch["load"][r] += share[r]
            batches.append(batch)
            mb[i], first_rank[i], slot[i] = len(batches) - 1, 0, 0
    return {"cp_size": cp, "micro_batch": mb, "group_rank": first_rank, "slot": slot,
            "n_micro_batches": len(batches)}
