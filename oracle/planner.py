"""Page-table planner, step by step, in integers (TEST INFRASTRUCTURE ONLY).

KPage paper, section 3.2 (forward page walk, Q64/Q128 routes, validity masks),
section 3.3 (K/V owners, reverse-Q neighbourhoods, Q pages, page-pair adjacency),
section 3.4 (metadata built from the graph and valid-row counts only) and
section 4.4 (physical pair-capacity accounting).  The equations of those
sections are missing from the text; the readings taken here:

  pages          p_b = ceil(c_b / 16); page j of block b is row range
                 [o_b + 16 j, o_b + 16 j + 16), page id o_b / 16 + j
  route          c_q = 0 skipped; 1..64 -> M64 x N256 (16 pages per step);
                 65..128 -> M128 x N128 (8 pages per step)
  forward walk   all full pages of K_q (K_q order, pages ascending), then the
                 partial tail page of each partial block (K_q order), then
                 dummy pages (id -1) up to a multiple of the pages per step
  validity       one 16-bit row mask per walk position (full 0xFFFF, tail
                 (1 << (c mod 16)) - 1, dummy 0); position 2i in the low half
                 and 2i+1 in the high half of 32-bit word i
  queues         per route, entries (b*H + h, q) by descending unpadded walk
                 length, then ascending b*H + h, then ascending q
  owners         8 page slots; each full block (c = 128) takes its own owner in
                 ascending block order; then the blocks with 0 < c < 128 fill
                 owners one at a time, never crossing an owner: the smallest
                 unplaced one opens an owner, and while one fits, the fitting
                 block adding the fewest query blocks to the owner's reverse
                 neighbourhood joins (ties to the smaller index); the aligned
                 flag is set when one block with 8 pages fills the owner
  reverse Q      bitmap[owner(k)][q] over the graph edges with c_q, c_k > 0;
                 each owner's list is its set bits in ascending q
  Q groups       q_group = 0: one group; q_group = n > 0: G_g = the Q blocks
                 [g n, (g + 1) n); the reverse neighbourhood of owner t in group
                 g is its list restricted to G_g (section 3.3.2), except that an
                 owner whose whole list holds at most n Q blocks is already within
                 the bound the grouping serves and keeps its list whole in group 0.
                 Tables are kept per (owner, group) pair, owner-major, empty pairs
                 included
  Q-page walk    per (owner, group): pages 8q + j of full Q blocks in the list,
                 then the pages of partial Q blocks, then dummies up to a
                 multiple of 8
  adjacency      per 8-page step, bit 8 j + i set when Q slot j and K slot i are
                 real pages whose blocks form a graph edge
  backward order work items (b*H + h, owner, group) for every pair with a
                 non-empty group list, plus (b*H + h, owner, 0) for an owner whose
                 lists are all empty (it still writes its zero gradients); by
                 descending step count, then ascending b*H + h, owner, group;
                 exported as (b*H + h, owner * n_groups + group)
  uncovered      K/V pages of [0, seq_kv / 16) inside no block's page footprint,
                 ascending: no query reaches their rows, so their dK, dV rows are
                 zero by definition and the backward writes them as such
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np

PAGE = 16
BLOCK = 128
FULL_MASK = 0xFFFF


def _pages(c: int) -> int:
    return -(-c // PAGE)


def _tail_mask(c: int) -> int:
    t = c % PAGE
    return (1 << t) - 1


@dataclass
class PlanTables:
    # forward (per graph slot, concatenated over slots)
    fwd_route: np.ndarray          # int32 [G, n_q]  0 / 64 / 128
    fwd_walk_ptr: np.ndarray       # int64 [G, n_q + 1] absolute offsets into fwd_walk
    fwd_walk: np.ndarray           # int32 page ids, -1 = dummy
    fwd_nfull: np.ndarray          # int32 [G, n_q]
    fwd_valid: np.ndarray          # uint32, word i of a walk at fwd_walk_ptr / 2 + i
    q64_queue: np.ndarray          # int32 [n, 2] (bh, q)
    q128_queue: np.ndarray         # int32 [n, 2]
    # backward
    owner_ptr: np.ndarray          # int64 [G + 1] offsets into owners
    owners: np.ndarray             # int32 [n_own, 8] page ids, -1 = empty slot
    owner_aligned: np.ndarray      # uint8 [n_own]
    revq_ptr: np.ndarray           # int64 [n_own * n_groups + 1] per (owner, group)
    revq: np.ndarray               # int32 Q block ids
    qwalk_ptr: np.ndarray          # int64 [n_own * n_groups + 1] offsets into qwalk (multiples of 8)
    qwalk: np.ndarray              # int32 Q page ids (8 q + j), -1 = dummy
    adj: np.ndarray                # uint64, step s of owner t at qwalk_ptr[t] / 8 + s
    bwd_queue: np.ndarray          # int32 [n, 2] (bh, owner index within its slot * n_groups + group)
    uncovered_ptr: np.ndarray      # int64 [G + 1] offsets into uncovered
    uncovered: np.ndarray          # int32 K/V page ids outside every block footprint
    stats: Dict[str, int] = field(default_factory=dict)


def _fwd_slot(c_q, c_k, o_k, rows, align64: int, align128: int):
    """Walks, routes, n_full and validity words of one graph slot."""
    routes, walks, nfull, masks = [], [], [], []
    for q, ks in enumerate(rows):
        cq = int(c_q[q])
        if cq == 0:
            routes.append(0)
            walks.append([])
            nfull.append(0)
            masks.append([])
            continue
        route = 64 if cq <= 64 else 128
        full, tails, tail_masks = [], [], []
        for k in ks:
            ck = int(c_k[k])
            base = int(o_k[k]) // PAGE
            for j in range(ck // PAGE):
                full.append(base + j)
            if ck % PAGE:
                tails.append(base + ck // PAGE)
                tail_masks.append(_tail_mask(ck))
        unpadded = full + tails
        per_step = align64 if route == 64 else align128
        pad = (-len(unpadded)) % per_step
        routes.append(route)
        walks.append(unpadded + [-1] * pad)
        nfull.append(len(full))
        masks.append([FULL_MASK] * len(full) + tail_masks + [0] * pad)
    return routes, walks, nfull, masks


def _owners_slot(c_k, o_k, c_q, rows):
    """Owners of one graph slot (section 3.3.1 says only that partial blocks are packed;
    reading R15): every full block (c = 128) is an owner of its own, in block order.  The
    partial blocks (0 < c < 128) then fill owners one at a time: the unplaced partial
    block of smallest index opens an owner; while some unplaced partial block fits into the
    owner's free slots, the one that adds the fewest query blocks to the owner's reverse
    neighbourhood joins it (ties to the smaller index), its pages after those already in
    the owner.  A block's reverse neighbourhood is the set of query blocks with c_q > 0
    that select it."""
    R = {k: set() for k in range(len(c_k))}
    for q, row in enumerate(rows):
        if int(c_q[q]) == 0:
            continue
        for k in row:
            if int(c_k[int(k)]) > 0:
                R[int(k)].add(q)
    owners, aligned, owner_of = [], [], {}
    for k in range(len(c_k)):
        if int(c_k[k]) == BLOCK:
            base = int(o_k[k]) // PAGE
            owner_of[k] = len(owners)
            owners.append([base + j for j in range(8)])
            aligned.append(1)
    left = [k for k in range(len(c_k)) if 0 < int(c_k[k]) < BLOCK]
    while left:
        seed = left.pop(0)
        t = len(owners)
        owners.append([])
        aligned.append(0)
        covered = set()

        def place(k):
            owner_of[k] = t
            base = int(o_k[k]) // PAGE
            owners[t].extend(base + j for j in range(_pages(int(c_k[k]))))
            covered.update(R[k])

        place(seed)
        while True:
            free = 8 - len(owners[t])
            best, best_new = None, None
            for k in left:
                if _pages(int(c_k[k])) <= free:
                    new_q = len(R[k] - covered)
                    if best_new is None or new_q < best_new:
                        best, best_new = k, new_q
            if best is None:
                break
            left.remove(best)
            place(best)
    for t, pages in enumerate(owners):
        if aligned[t] == 0 and len(pages) == 8:
            blocks = {owner_block for owner_block, ot in owner_of.items() if ot == t}
            if len(blocks) == 1:
                aligned[t] = 1
        pages.extend([-1] * (8 - len(pages)))
    return owners, aligned, owner_of


def oracle_plan(problem, align_q64: int = 16, align_q128: int = 8, q_group: int = 0) -> PlanTables:
    """Build every forward and backward table of ``problem`` (a workloads.Workload-like object)."""
    G, n_q = problem.q_valid.shape
    group_size = q_group if q_group > 0 else n_q
    n_groups = -(-n_q // group_size)
    H = problem.heads
    BH = problem.batch * H
    slots_bh = {}
    for bh in range(BH):
        slots_bh.setdefault(bh if problem.per_head else 0, []).append(bh)

    f_route = np.zeros((G, n_q), dtype=np.int32)
    f_ptr = np.zeros((G, n_q + 1), dtype=np.int64)
    f_nfull = np.zeros((G, n_q), dtype=np.int32)
    f_walk: List[int] = []
    f_valid: List[int] = []
    o_ptr = np.zeros(G + 1, dtype=np.int64)
    owners_all, aligned_all, revq_ptr, revq, qw_ptr, qwalk, adj = [], [], [0], [], [0], [], []
    unc_ptr, unc = [0], []
    steps_of: List[List[int]] = []
    stats = dict(useful=0, whole_block=0, paged_m128=0, nominal=0, scheduled=0,
                 bwd_physical=0, bwd_useful_check=0)
    unpadded_len = np.zeros((G, n_q), dtype=np.int64)

    for g in range(G):
        c_q, c_k, o_k = problem.q_valid[g], problem.kv_valid[g], problem.kv_offset[g]
        rows = [list(problem.q2k_idx[problem.q2k_ptr[g, q]:problem.q2k_ptr[g, q + 1]]) for q in range(n_q)]
        nbh = len(slots_bh.get(g, []))
        routes, walks, nfull, masks = _fwd_slot(c_q, c_k, o_k, rows, align_q64, align_q128)
        for q in range(n_q):
            f_route[g, q] = routes[q]
            f_nfull[g, q] = nfull[q]
            f_ptr[g, q] = len(f_walk)
            f_walk.extend(walks[q])
            m = masks[q]
            f_valid.extend(m[2 * i] | (m[2 * i + 1] << 16) for i in range(len(m) // 2))
            if routes[q]:
                unpadded_len[g, q] = sum(1 for x in walks[q] if x >= 0)
                cq = int(c_q[q])
                M = routes[q] if routes[q] == 64 else 128
                psum = sum(_pages(int(c_k[k])) for k in rows[q])
                stats["useful"] += nbh * sum(cq * int(c_k[k]) for k in rows[q])
                stats["whole_block"] += nbh * BLOCK * BLOCK * len(rows[q])
                stats["paged_m128"] += nbh * BLOCK * PAGE * psum
                stats["nominal"] += nbh * M * PAGE * psum
                stats["scheduled"] += nbh * M * PAGE * len(walks[q])
        f_ptr[g, n_q] = len(f_walk)

        # backward: owners, reverse Q, Q-page walks, adjacency
        owners, aligned, owner_of = _owners_slot(c_k, o_k, c_q, rows)
        o_ptr[g + 1] = o_ptr[g] + len(owners)
        page_block = {}
        for k, t in owner_of.items():
            for j in range(_pages(int(c_k[k]))):
                page_block[int(o_k[k]) // PAGE + j] = k
        unc.extend(pg for pg in range(int(problem.seq_kv) // PAGE) if pg not in page_block)
        unc_ptr.append(len(unc))
        kmask = {}
        for k in owner_of:
            ck = int(c_k[k])
            for j in range(_pages(ck)):
                kmask[int(o_k[k]) // PAGE + j] = FULL_MASK if (j + 1) * PAGE <= ck else _tail_mask(ck)
        edges = set()
        bitmap = np.zeros((len(owners), n_q), dtype=bool)
        for q in range(n_q):
            if int(c_q[q]) == 0:
                continue
            for k in rows[q]:
                if int(c_k[k]) == 0:
                    continue
                edges.add((q, int(k)))
                bitmap[owner_of[int(k)], q] = True
        slot_steps = []  # [owner][group]
        for t, pages in enumerate(owners):
            R_all = [int(x) for x in np.nonzero(bitmap[t])[0]]
            split = len(R_all) > group_size  # a list of at most n Q blocks stays whole
            owner_steps = []
            for grp in range(n_groups):
                if split:
                    R = [q for q in R_all if q // group_size == grp]
                else:
                    R = R_all if grp == 0 else []
                revq.extend(R)
                revq_ptr.append(len(revq))
                qp = [8 * q + j for q in R if int(c_q[q]) == BLOCK for j in range(8)]
                qp += [8 * q + j for q in R if 0 < int(c_q[q]) < BLOCK for j in range(_pages(int(c_q[q])))]
                qp += [-1] * ((-len(qp)) % 8)
                qwalk.extend(qp)
                qw_ptr.append(len(qwalk))
                n_steps = len(qp) // 8
                owner_steps.append(n_steps)
                for s in range(n_steps):
                    word = 0
                    for j in range(8):
                        qpg = qp[8 * s + j]
                        if qpg < 0:
                            continue
                        qb = qpg // 8
                        cq = int(c_q[qb])
                        qm = FULL_MASK if ((qpg % 8) + 1) * PAGE <= cq else _tail_mask(cq)
                        for i in range(8):
                            kpg = pages[i]
                            if kpg < 0:
                                continue
                            if (qb, page_block[kpg]) in edges:
                                word |= 1 << (8 * j + i)
                                stats["bwd_useful_check"] += nbh * bin(qm).count("1") * bin(kmask[kpg]).count("1")
                    adj.append(word)
                stats["bwd_physical"] += nbh * BLOCK * BLOCK * n_steps
            slot_steps.append(owner_steps)
            owners_all.append(pages)
            aligned_all.append(aligned[t])
        steps_of.append(slot_steps)

    def _queue(route):
        ent = []
        for bh in range(BH):
            g = bh if problem.per_head else 0
            for q in range(n_q):
                if f_route[g, q] == route:
                    ent.append((-int(unpadded_len[g, q]), bh, q))
        ent.sort()
        return np.asarray([(bh, q) for _, bh, q in ent], dtype=np.int32).reshape(-1, 2)

    def revq_len(g, t, grp):
        i = (int(o_ptr[g]) + t) * n_groups + grp
        return revq_ptr[i + 1] - revq_ptr[i]

    bq = []
    for bh in range(BH):
        g = bh if problem.per_head else 0
        for t, owner_steps in enumerate(steps_of[g]):
            # a group with no Q block of the owner's neighbourhood has no work; an owner with none
            # at all keeps one item for group 0
            groups = [grp for grp in range(n_groups) if revq_len(g, t, grp) > 0] or [0]
            for grp in groups:
                bq.append((-owner_steps[grp], bh, t, grp))
    bq.sort()

    return PlanTables(
        fwd_route=f_route, fwd_walk_ptr=f_ptr, fwd_walk=np.asarray(f_walk, dtype=np.int32),
        fwd_nfull=f_nfull, fwd_valid=np.asarray(f_valid, dtype=np.uint32),
        q64_queue=_queue(64), q128_queue=_queue(128),
        owner_ptr=o_ptr, owners=np.asarray(owners_all, dtype=np.int32).reshape(-1, 8),
        owner_aligned=np.asarray(aligned_all, dtype=np.uint8),
        revq_ptr=np.asarray(revq_ptr, dtype=np.int64), revq=np.asarray(revq, dtype=np.int32),
        qwalk_ptr=np.asarray(qw_ptr, dtype=np.int64), qwalk=np.asarray(qwalk, dtype=np.int32),
        adj=np.asarray(adj, dtype=np.uint64),
        bwd_queue=np.asarray([(bh, t * n_groups + grp) for _, bh, t, grp in bq], dtype=np.int32).reshape(-1, 2),
        uncovered_ptr=np.asarray(unc_ptr, dtype=np.int64), uncovered=np.asarray(unc, dtype=np.int32),
        stats=stats,
    )
