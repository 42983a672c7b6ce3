"""Pins of the oracle's paging arithmetic to the numbers the paged-KV page prints.

Fixture: tests/golden/paged_kv_worked_example.json (each block cites its section
of the paged-KV page, "KV cache phân trang, hay vì sao đặt trước theo độ dài
tối đa là hoang phí").
"""
import json
import os

import numpy as np
import pytest

from oracle import paging

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "paged_kv_worked_example.json")))
T = GOLD["table"]
LENS, P, R = T["lens"], T["page_size"], T["reserve"]


def test_table_rows():
    acc = paging.page_accounting(LENS, P, R)
    for i, row in enumerate(T["rows"]):
        assert acc["pages"][i] == row["pages"]
        assert acc["held"][i] == row["held"]
        assert acc["last_fill"][i] == row["last_fill"]
        assert acc["slack"][i] == row["slack"]
        assert acc["naive_held"][i] == row["naive_held"]
        assert acc["naive_waste"][i] == row["naive_waste"]


def test_table_totals():
    acc = paging.page_accounting(LENS, P, R)
    t = T["total"]
    assert acc["total_used"] == t["used"]
    assert acc["total_pages"] == t["pages"]
    assert acc["total_held"] == t["held"]
    assert acc["full_last_pages"] == t["full_last_pages"]
    assert acc["total_slack"] == t["slack"]
    assert acc["total_naive_held"] == t["naive_held"]
    assert acc["total_naive_waste"] == t["naive_waste"]


def test_fragmentation_figures():
    f = GOLD["fragmentation"]
    acc = paging.page_accounting(LENS, P, R, bytes_per_token=f["bytes_per_token"])
    assert acc["total_naive_held"] == f["naive_held"]
    assert acc["total_naive_waste"] == f["naive_waste"]
    assert round(100 * acc["naive_waste_frac"], 1) == f["naive_waste_pct"]
    assert round(acc["naive_waste_mib"], 1) == f["naive_waste_mib"]
    assert round(acc["naive_held_mib"], 1) == f["naive_held_mib"]
    cells, dashed = paging.naive_page_grid(LENS, P, R)
    assert (cells, dashed) == (f["grid_cells"], f["grid_dashed"])


def test_paging_section():
    g = GOLD["paging"]
    acc = paging.page_accounting(LENS, P, R, bytes_per_token=GOLD["fragmentation"]["bytes_per_token"])
    assert acc["pages"] == g["pages"]
    assert acc["total_pages"] == g["total_pages"]
    assert acc["total_held"] == g["held"]
    assert round(acc["paged_held_mib"], 1) == g["paged_held_mib"]
    assert acc["slack"][0] == g["first_request_tail"]
    assert acc["total_slack"] == g["total_slack"]
    assert round(100 * acc["paged_waste_frac"], 1) == g["paged_waste_pct"]
    inv = g["invariant"]
    assert acc["total_used"] + acc["total_slack"] == acc["total_pages"] * P == inv["held"]
    assert (inv["used"], inv["slack"], inv["pages"], inv["page_size"]) == (946, 30, 61, 16)


def test_page_size_special_cases():
    g = GOLD["paging"]
    acc1 = paging.page_accounting(LENS, 1, R)
    assert acc1["total_slack"] == g["page_size_1_slack"]
    acc512 = paging.page_accounting(LENS, 512, R)
    assert acc512["total_held"] == g["page_size_512_held"] == acc512["total_naive_held"]
    assert round(100 * acc512["paged_waste_frac"], 1) == g["page_size_512_waste_pct"]


@pytest.mark.parametrize("P_", [1, 2, 3, 7, 16, 64, 100, 512, 1000])
def test_invariant_any_page_size(P_):
    rng = np.random.default_rng(P_)
    lens = rng.integers(1, 5000, size=40).tolist()
    acc = paging.page_accounting(lens, P_, 5000)
    assert acc["total_used"] + acc["total_slack"] == acc["total_pages"] * P_
    assert all(0 <= s < P_ for s in acc["slack"])
    assert all(1 <= f <= P_ for f in acc["last_fill"])


def test_capacity_section():
    c = GOLD["capacity"]
    cap = paging.admission_capacity(c["pool_bytes"], c["bytes_per_token"], LENS, P, R)
    assert cap["slots"] == c["slots"]
    assert cap["naive"] == c["naive_requests"]
    assert cap["paged"] == c["paged_requests"]
    assert round(cap["mean_cost"], 1) == c["paged_mean_slots"]
    assert round(cap["paged"] / cap["naive"], 1) == c["ratio"]
    assert cap["full_rounds"] == c["full_rounds"]
    assert cap["left_after_rounds"] == c["left_after_rounds"] == sum(c["last_round_costs"])
    assert cap["paged"] - cap["full_rounds"] * len(LENS) == c["admitted_in_last_round"]
    acc = paging.page_accounting(LENS, P, R)
    assert acc["held"][cap["blocked_request"]] == c["blocked_request_cost"]
    assert cap["left_at_stop"] < c["blocked_request_cost"]


def test_sharing_section_formula():
    s = GOLD["sharing"]
    assert paging.prefix_pages_saved(s["requests"], s["prefix_len"], P) == s["saved_pages"]
    assert s["saved_pages"] * P == s["saved_tokens"]
    assert paging.prefix_pages_saved(s["requests"], 15, P) == s["prefix_15_saved"]
    assert paging.prefix_pages_saved(s["requests"], 16, P) == s["prefix_16_saved"]
    assert paging.prefix_pages_saved(1, 1000, P) == 0          # one copy must remain


def test_sharing_section_tables():
    """The allocation policy realises the formula: 976 tokens held drop to 848."""
    s = GOLD["sharing"]
    grp = np.array([0, 0, 0, -1, -1])
    out = paging.build_page_tables(LENS, P, np.arange(70), grp, [s["prefix_len"]])
    assert out["saved"] == s["saved_pages"]
    assert out["pages_in_use"] * P == s["held_after"]
    assert (61 - out["pages_in_use"]) * P == s["saved_tokens"]
    tab = out["table"]
    # the three members point at the same 4 full prefix pages, and nothing else is shared
    assert (tab[0, :4] == tab[1, :4]).all() and (tab[0, :4] == tab[2, :4]).all()
    assert len(set(tab[0, 4:26]) & set(tab[1, 4:6])) == 0
    assert (out["refcount"][tab[0, :4]] == 3).all()
    assert out["refcount"].max() == 3
    # prefix of 15 tokens shares nothing; 16 shares one page per member
    assert paging.build_page_tables(LENS, P, np.arange(70), grp, [15])["pages_in_use"] == 61
    assert paging.build_page_tables(LENS, P, np.arange(70), grp, [16])["pages_in_use"] == 59


def test_quiz_by_formula():
    """Quiz at the end of the paged-KV page; its answers are not printed, these follow the
    two formulas the page closes with (ceil for allocation, (n-1)*floor for sharing)."""
    assert paging.pages_needed(100, 16) == 7 and paging.slack(100, 16) == 12
    assert paging.prefix_pages_saved(4, 40, 16) == 6


def test_tables_ascending_policy():
    out = paging.build_page_tables(LENS, P, np.arange(66))
    tab, n = out["table"], out["num_pages"]
    assert n.tolist() == [26, 6, 16, 2, 11]
    # ascending free order, requests in order, logical pages in order
    flat = np.concatenate([tab[i, :n[i]] for i in range(5)])
    assert flat.tolist() == list(range(61))
    assert (tab[1, 6:] == -1).all()
    assert out["free"] == list(range(61, 66))


def test_tables_permuted_policy():
    perm = np.random.default_rng(3).permutation(100)
    out = paging.build_page_tables(LENS, P, perm)
    n = out["num_pages"]
    flat = np.concatenate([out["table"][i, :n[i]] for i in range(5)])
    assert flat.tolist() == perm[:61].tolist()
    assert (out["refcount"][perm[:61]] == 1).all() and out["refcount"].sum() == 61


def test_tables_out_of_pages_and_errors():
    with pytest.raises(MemoryError):
        paging.build_page_tables(LENS, P, np.arange(60))
    with pytest.raises(ValueError):
        paging.build_page_tables(LENS, P, [0, 0, 1])
    with pytest.raises(ValueError):
        paging.build_page_tables([10, 20], P, np.arange(10), [0, 0], [16])   # shorter than prefix
    with pytest.raises(ValueError):
        paging.build_page_tables(LENS, P, np.arange(70), max_pages=10)


def test_workload_prefix_saving():
    """128 requests sharing a 16384-token prefix at page size 64 save 127 x 256 pages."""
    lens = 16384 + np.random.default_rng(0).integers(1024, 4097, size=128)
    out = paging.build_page_tables(lens, 64, np.arange(8576), np.zeros(128, int), [16384],
                                   max_pages=320)
    assert out["saved"] == 127 * 256 == 32512
    need = sum(paging.pages_needed(int(L), 64) for L in lens)
    assert out["pages_in_use"] == need - 32512


def test_grow():
    out = paging.build_page_tables([16, 17], 16, np.arange(8))
    g = paging.grow_page_tables(out["table"], out["num_pages"], [17, 17], 16, out["free"])
    assert g["num_pages"].tolist() == [2, 2]
    assert g["table"][0, 1] == out["free"][0]
    with pytest.raises(MemoryError):
        paging.grow_page_tables(out["table"], out["num_pages"], [32, 32], 16, [])
    with pytest.raises(ValueError):
        paging.grow_page_tables(out["table"], out["num_pages"], [0, 17], 16, out["free"])


def test_grow_several_requests_by_hand():
    """Three requests grown at once, worked by hand from the allocation reading (requests in
    index order, each one's new logical pages in order, popped from the front of the free
    list).  Lengths 16 / 17 / 5 at P = 16 hold 1 / 2 / 1 pages: free order 7 3 5 1 0 2 6 4
    gives request 0 page 7, request 1 pages 3 and 5, request 2 page 1, leaving 0 2 6 4.
    Growing to 33 / 17 / 40 tokens needs 3 / 2 / 3 pages: request 0 takes 0 and 2, request 1
    nothing, request 2 takes 6 and 4.  A round-robin or per-page-index order would give
    request 0 pages 0 and 6 instead."""
    free = np.array([7, 3, 5, 1, 0, 2, 6, 4])
    out = paging.build_page_tables([16, 17, 5], 16, free, max_pages=3)
    assert out["table"].tolist() == [[7, -1, -1], [3, 5, -1], [1, -1, -1]]
    assert list(out["free"]) == [0, 2, 6, 4]
    g = paging.grow_page_tables(out["table"], out["num_pages"], [33, 17, 40], 16, out["free"])
    assert g["table"].tolist() == [[7, 0, 2], [3, 5, -1], [1, 6, 4]]
    assert g["num_pages"].tolist() == [3, 2, 3] and list(g["free"]) == []
    # one page more than the pool has left (request 1 to 3 pages): refused, tables unchanged
    with pytest.raises(MemoryError):
        paging.grow_page_tables(g["table"], g["num_pages"], [33, 33, 40], 16, g["free"])
    assert g["table"].tolist() == [[7, 0, 2], [3, 5, -1], [1, 6, 4]]


def test_physical_slot():
    out = paging.build_page_tables(LENS, P, np.arange(66)[::-1].copy())
    assert paging.physical_slot(out["table"], 0, 0, P) == 65 * 16
    assert paging.physical_slot(out["table"], 1, 17, P) == (65 - 27) * 16 + 1
