"""Paging arithmetic and page tables (oracle; test infrastructure only).

Source: the paged-KV page, "KV cache phân trang, hay vì sao đặt trước theo độ
dài tối đa là hoang phí".  Sections used:

* opening table and "Phân mảnh trong, và nó lớn cỡ nào": the naive scheme
  reserves the maximum length R for every request; waste = held - used.
* "Phân trang: bỏ luôn ràng buộc liền mạch": pages = ceil(length / page_size);
  the slack of a request is the empty tail of its last page; used tokens plus
  every last-page slack equals pages x page_size.
* "Con số thật sự đáng quan tâm": a pool of slots (bytes / bytes-per-token);
  naive admits floor(slots / R) requests; the paged count admits the request
  list over and over in list order until one no longer fits.
* "Chia sẻ trang": requests with a common prefix point their page tables at
  the same pages; only full prefix pages can be shared, one copy must remain:
  saved = (n - 1) * floor(prefix / page_size).

The pages do not say how physical pages are chosen.  The reading used here
(and stated as the allocation policy of the library) is:

1. the pool hands out physical page ids in a given ``free_order`` (ascending,
   or a seeded permutation), popping from the front;
2. requests are built in index order, each one's logical pages in order;
3. the full prefix pages of a sharing group are popped when the group's first
   member is built; later members point at the same ids (refcount = members);
4. the page holding the end of the prefix and the first private token, and
   every later page, is private;
5. unused table entries are -1.
"""
from __future__ import annotations

import numpy as np


def pages_needed(length: int, page_size: int) -> int:
    """ceil(length / page_size) ("Phân trang" section)."""
    return -(-int(length) // int(page_size))


def last_page_fill(length: int, page_size: int) -> int:
    """Tokens stored in the last page (the "trang cuối" column of the table)."""
    n = pages_needed(length, page_size)
    return int(length) - (n - 1) * int(page_size) if n else 0


def slack(length: int, page_size: int) -> int:
    """Empty tail of the last page (the "thừa" column)."""
    return pages_needed(length, page_size) * int(page_size) - int(length)


def page_accounting(lens, page_size: int, reserve: int, bytes_per_token: int | None = None) -> dict:
    """Per-request and total accounting of the opening table.

    Returns pages, paged tokens held, last-page fill, slack, naive held and
    naive waste per request, their totals, the two waste fractions and, when
    ``bytes_per_token`` is given, the MiB figures of the fragmentation section.
    Requests longer than ``reserve`` do not fit the naive scheme; they are
    reported in ``naive_overflow`` (the page does not cover that case).
    """
    lens = [int(x) for x in lens]
    P, R = int(page_size), int(reserve)
    pages = [pages_needed(L, P) for L in lens]
    held = [n * P for n in pages]
    fill = [last_page_fill(L, P) for L in lens]
    sl = [slack(L, P) for L in lens]
    naive_held = [R] * len(lens)
    naive_waste = [R - L for L in lens]
    out = dict(
        pages=pages, held=held, last_fill=fill, slack=sl,
        naive_held=naive_held, naive_waste=naive_waste,
        naive_overflow=[i for i, L in enumerate(lens) if L > R],
        total_used=sum(lens), total_pages=sum(pages), total_held=sum(held),
        total_slack=sum(sl), full_last_pages=sum(1 for f in fill if f == P),
        total_naive_held=sum(naive_held), total_naive_waste=sum(naive_waste),
    )
    out["paged_waste_frac"] = out["total_slack"] / out["total_held"] if out["total_held"] else 0.0
    out["naive_waste_frac"] = (out["total_naive_waste"] / out["total_naive_held"]
                               if out["total_naive_held"] else 0.0)
    if bytes_per_token is not None:
        mib = float(bytes_per_token) / float(1 << 20)
        out["paged_held_mib"] = out["total_held"] * mib
        out["naive_held_mib"] = out["total_naive_held"] * mib
        out["naive_waste_mib"] = out["total_naive_waste"] * mib
    return out


def naive_page_grid(lens, page_size: int, reserve: int) -> tuple[int, int]:
    """(cells, reserved-but-empty cells) of the naive grid drawn with paged cells.

    Every request reserves R / page_size cells; a cell holding any token of
    the request is used, the rest are drawn dashed.
    """
    per = int(reserve) // int(page_size)
    cells = per * len(list(lens))
    used = sum(pages_needed(L, page_size) for L in lens)
    return cells, cells - used


def prefix_pages_saved(n_requests: int, prefix_len: int, page_size: int) -> int:
    """(n - 1) * floor(prefix / page_size) ("Chia sẻ trang" section)."""
    if n_requests <= 0:
        return 0
    return (int(n_requests) - 1) * (int(prefix_len) // int(page_size))


def admission_capacity(pool_bytes: int, bytes_per_token: int, lens, page_size: int,
                       reserve: int) -> dict:
    """How many requests one pool holds, naive vs paged ("Con số thật sự..." section).

    Slots are tokens of cache.  Naive: every request costs ``reserve`` slots.
    Paged: a request costs pages x page_size slots; requests arrive over and
    over in list order, never finish, and are admitted until the first one that
    does not fit.
    """
    slots = int(pool_bytes) // int(bytes_per_token)
    naive = slots // int(reserve)
    cost = [pages_needed(L, page_size) * int(page_size) for L in lens]
    left, admitted, i = slots, 0, 0
    rounds = 0
    while cost[i] <= left:
        left -= cost[i]
        admitted += 1
        i += 1
        if i == len(cost):
            i = 0
            rounds += 1
    return dict(slots=slots, naive=naive, paged=admitted, mean_cost=sum(cost) / len(cost),
                full_rounds=rounds, left_after_rounds=slots - rounds * sum(cost),
                left_at_stop=left, blocked_request=i)


def build_page_tables(lens, page_size: int, free_order, prefix_group=None,
                      prefix_len_of_group=None, max_pages: int | None = None) -> dict:
    """Page tables under the allocation policy in the module docstring.

    ``prefix_group[i]`` is the sharing group of request i (-1 = none) and
    ``prefix_len_of_group[g]`` that group's prefix length in tokens.  Returns
    the table [n, max_pages] (int32, -1 padded), pages per request, the
    refcount of every physical page, pages saved by sharing and the free list
    left over.  Raises ``MemoryError`` when the pool runs out (the caller sees
    no partial table), ``ValueError`` on inconsistent input.
    """
    lens = [int(x) for x in lens]
    n = len(lens)
    P = int(page_size)
    free = [int(x) for x in free_order]
    num_pool = len(free)
    if sorted(free) != list(range(num_pool)):
        raise ValueError("free_order must be a permutation of 0..num_pages-1")
    need = [pages_needed(L, P) for L in lens]
    if max_pages is None:
        max_pages = max(need) if need else 0
    if any(x > max_pages for x in need):
        raise ValueError("a request needs more pages than max_pages")
    groups = [-1] * n if prefix_group is None else [int(g) for g in prefix_group]
    shared_count = {}  # group -> number of full prefix pages
    for i, g in enumerate(groups):
        if g < 0:
            continue
        p = int(prefix_len_of_group[g])
        if lens[i] < p:
            raise ValueError("a request is shorter than its group's prefix")
        shared_count[g] = p // P

    table = np.full((n, max_pages), -1, dtype=np.int32)
    refcount = np.zeros(num_pool, dtype=np.int64)
    shared_ids = {}  # group -> list of physical ids of its full prefix pages
    head = 0
    for i in range(n):
        g = groups[i]
        for j in range(need[i]):
            if g >= 0 and j < shared_count[g]:
                ids = shared_ids.setdefault(g, [])
                if j < len(ids):          # a later member: point at the group's page
                    table[i, j] = ids[j]
                    refcount[ids[j]] += 1
                    continue
                if head == num_pool:
                    raise MemoryError("pool out of pages")
                ids.append(free[head])
            elif head == num_pool:
                raise MemoryError("pool out of pages")
            pid = free[head]
            head += 1
            table[i, j] = pid
            refcount[pid] += 1
    members = {}
    for g in groups:
        if g >= 0:
            members[g] = members.get(g, 0) + 1
    saved = sum(prefix_pages_saved(members[g], int(prefix_len_of_group[g]), P) for g in members)
    return dict(table=table, num_pages=np.asarray(need, dtype=np.int32), refcount=refcount,
                saved=saved, free=free[head:], pages_in_use=head)


def physical_slot(table: np.ndarray, req: int, pos: int, page_size: int) -> int:
    """Physical token slot of logical position ``pos`` of request ``req``."""
    page = int(table[req, pos // page_size])
    if page < 0:
        raise IndexError("position not covered by the page table")
    return page * page_size + pos % page_size


def grow_page_tables(table: np.ndarray, num_pages, new_lens, page_size: int, free) -> dict:
    """Give each request the pages its new length needs, popping ``free`` in order.

    Requests are served in index order, new logical pages in order (the same
    policy as ``build_page_tables``).  Lengths may not shrink.  Raises
    ``MemoryError`` (no partial change) when the pool runs out.
    """
    table = np.array(table, dtype=np.int32, copy=True)
    have = [int(x) for x in num_pages]
    free = [int(x) for x in free]
    want = [pages_needed(L, page_size) for L in new_lens]
    if any(w < h for w, h in zip(want, have)):
        raise ValueError("a length shrank")
    if any(w > table.shape[1] for w in want):
        raise ValueError("a request needs more pages than max_pages")
    if sum(w - h for w, h in zip(want, have)) > len(free):
        raise MemoryError("pool out of pages")
    head = 0
    for i, (h, w) in enumerate(zip(have, want)):
        for j in range(h, w):
            table[i, j] = free[head]
            head += 1
    return dict(table=table, num_pages=np.asarray(want, dtype=np.int32), free=free[head:])
