"""Pins of the oracle's closed forms against figures the pages print."""

import json
import os

import pytest

from oracle import sizes


@pytest.fixture(scope="module")
def figures(golden_dir):
    with open(os.path.join(golden_dir, "page_figures.json")) as f:
        return {e["name"]: e for e in json.load(f)["entries"]}


def _close(got, entry):
    want = entry["value"]
    if "tolerance_rel" in entry:
        return abs(got - want) <= entry["tolerance_rel"] * want
    return got == want


def test_bytes_per_token(figures):
    for name in ("kv_bytes_per_token_7b", "kv_bytes_per_token_per_layer", "kv_bytes_per_token_per_layer_int8"):
        e = figures[name]
        a = e["args"]
        got = sizes.kv_bytes_per_token(a["layers"], a["heads"], a["head_dim"], a["dtype_bytes"])
        assert _close(got, e), (name, got)
    for name in ("kv_bytes_per_token_7b_hidden", "kv_bytes_per_token_13b_hidden"):
        e = figures[name]
        a = e["args"]
        got = sizes.kv_bytes_per_token_hidden(a["layers"], a["hidden"], a["dtype_bytes"])
        assert _close(got, e), (name, got)
    # 13B: exactly 800 KiB, which the page rounds to "about 800KB".
    assert sizes.kv_bytes_per_token_hidden(40, 5120, 2) == 800 * 1024


def test_request_and_page_bytes(figures):
    for name in ("request_4096_tokens_7b_bytes", "request_2048_tokens_7b_bytes", "page_bytes_256_tokens"):
        e = figures[name]
        a = e["args"]
        assert a["tokens"] * a["bytes_per_token"] == e["value"]
        assert sizes.block_bytes(a["tokens"], a["bytes_per_token"]) == e["value"]
    e = figures["block_bytes_16_tokens_7b"]
    assert sizes.block_bytes(e["args"]["block_size"], e["args"]["bytes_per_token"]) == e["value"] == sizes.mib(8)
    e = figures["table_bytes_1M_entries"]
    assert sizes.table_bytes(e["args"]["entries"], e["args"]["entry_bytes"]) == e["value"]


def test_pool_capacity(figures):
    e = figures["usable_bytes_80GB_card_gib"]
    a = e["args"]
    assert a["total"] - a["weights"] - a["activations"] - a["framework"] == e["value"]
    e = figures["pool_blocks_80GB_card"]
    a = e["args"]
    nb = sizes.pool_blocks(sizes.gib(a["usable_gib"]), a["block_size"], a["bytes_per_token"])
    assert nb == e["value"]
    assert sizes.pool_token_capacity(nb, 16) == figures["pool_tokens_80GB_card"]["value"]
    assert sizes.max_requests(nb, 16, 500) == figures["max_requests_500_tokens"]["value"]
    # The page's 7168 needs binary units: decimal GB would give a different count.
    assert sizes.pool_blocks(56 * 10**9, 16, 524288) != 7168


def test_a100_page_count(figures):
    e = figures["a100_pages_256_tokens"]
    a = e["args"]
    pages = sizes.pool_blocks(a["hbm_bytes"], a["page_tokens"], a["bytes_per_token"])
    assert _close(pages, e), pages
    assert abs(pages * (1 - a["reserve"]) - a["after_reserve"]) <= e["tolerance_rel"] * a["after_reserve"]


def test_table_entries(figures):
    e = figures["table_entries_2048_tokens"]
    for bs, want in e["value"].items():
        assert sizes.blocks_for_length(2048, int(bs)) == want


def test_tail_waste(figures):
    e = figures["tail_waste_percent_mean_300"]
    for bs, want in e["value"].items():
        got = 100.0 * sizes.expected_tail_waste_fraction(int(bs), 300)
        assert abs(got - want) <= e["tolerance_abs_percent"], (bs, got, want)


@pytest.mark.parametrize("bs", [1, 4, 8, 16, 32, 64])
def test_fragmentation_brute_force(bs):
    # Over every length 1..k*bs the tail residues are uniform, so the mean
    # waste is exactly (bs - 1) / 2 slots: "about half a block".
    k = 7
    lengths = range(1, k * bs + 1)
    total = sizes.fragmentation_tokens(lengths, bs)
    assert total * 2 == (bs - 1) * k * bs
    # Brute force: count unused slots one by one.
    brute = 0
    for length in lengths:
        used = 0
        blocks = 0
        while used < length:
            blocks += 1
            used += bs
        brute += blocks * bs - length
    assert brute == total


def test_fragmentation_special_cases():
    # 4096 is a multiple of 8, 16 and 32: no waste; one token more wastes bs - 1.
    for bs in (8, 16, 32):
        assert sizes.fragmentation_tokens([4096] * 16, bs) == 0
        assert sizes.fragmentation_tokens([4097], bs) == bs - 1
    assert sizes.blocks_for_length(0, 16) == 0
    with pytest.raises(ValueError):
        sizes.blocks_for_length(-1, 16)


def test_unique_vs_logical_bytes():
    # Two sequences sharing their first block count it once in unique bytes.
    tables = [[5, 1], [5, 2]]
    lens = [20, 18]
    logical = sizes.logical_kv_bytes(lens, 2, 4, 2)
    unique = sizes.unique_kv_bytes(tables, lens, 16, 2, 4, 2)
    per = 2 * 2 * 4 * 2
    assert logical == 38 * per
    assert unique == (16 + 4 + 2) * per
