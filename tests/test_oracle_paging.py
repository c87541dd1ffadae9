"""Pins of the oracle's paging arithmetic against the pages' worked examples."""
import numpy as np

from oracle import attention as A
from tests.conftest import load_golden


def test_page_table_example():
    g = load_golden("page_table_example.json")
    lens = A.kv_lengths(g["kv_indptr"], g["last_page_len"], g["page_size"])
    assert lens.tolist() == g["expected_kv_len"]
    for i, rows in enumerate(g["expected_rows"]):
        got = A.physical_rows(g["kv_indptr"], g["kv_indices"], g["last_page_len"], g["page_size"], i)
        assert got.tolist() == rows


def test_token_address_example():
    g = load_golden("token_address.json")
    P = g["page_size"]
    n_pages = len(g["indices"])
    rows = A.physical_rows([0, n_pages], g["indices"], [P], P, 0)
    assert rows[g["logical_token"]] == g["expected_physical_token"]


def test_toy_bsr_rows():
    g = load_golden("toy_bsr_rows.json")
    rp = g["row_ptr"]
    last = [1] * (len(rp) - 1)
    for t, pages in enumerate(g["expected_pages_per_tile"]):
        assert A.physical_rows(rp, g["col_indices"], last, g["page_size"], t).tolist() == pages


def test_empty_request_has_no_rows():
    assert A.kv_lengths([0, 0, 2], [0, 3], 4).tolist() == [0, 7]
    assert A.physical_rows([0, 0, 2], [1, 0], [0, 3], 4, 0).size == 0
