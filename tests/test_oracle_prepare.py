"""Pins for the block-preparation reference (CPU only): the hand-worked
example of the DFlash block fill and the slot rule, and the capacity / slot
error conditions."""
import json
import os

import numpy as np

import oracle
from oracle.prepare import ERR_CAPACITY, ERR_SLOT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fx():
    return json.load(open(os.path.join(GOLDEN, "prepare_block_small.json")))


def test_golden_draft_pass():
    fx = _fx()
    ids, pos, loc, err = oracle.prepare_block(
        np.array(fx["verified_id"]), np.array(fx["seq_lens"]), np.array(fx["page_table"]),
        fx["page_size"], fx["block"], fx["mask_token_id"])
    e = fx["expect_draft_pass"]
    assert err == 0
    assert ids.tolist() == e["block_ids"]
    assert pos.tolist() == e["positions"]
    assert loc.tolist() == e["cache_loc"]


def test_golden_verify_pass():
    fx = _fx()
    ids, pos, loc, err = oracle.prepare_block(
        np.array(fx["verified_id"]), np.array(fx["seq_lens"]), np.array(fx["page_table"]),
        fx["page_size"], fx["block"], fx["mask_token_id"], np.array(fx["draft_tokens"]))
    assert err == 0
    assert ids.tolist() == fx["expect_verify_pass"]["block_ids"]
    assert loc.tolist() == fx["expect_draft_pass"]["cache_loc"]


def test_identity_table_gives_contiguous_slots():
    P, B = 16, 8
    L = np.array([0, 5, 31, 100])
    need = (L + 2 * B + P - 1) // P
    table = np.full((4, need.max()), -1)
    base = np.concatenate([[0], np.cumsum(need)[:-1]])
    for b in range(4):
        table[b, :need[b]] = base[b] + np.arange(need[b])
    _, pos, loc, err = oracle.prepare_block(np.zeros(4), L, table, P, B, 0)
    assert err == 0
    for b in range(4):
        assert loc[b].tolist() == list(base[b] * P + L[b] + np.arange(B))


def test_capacity_and_slot_errors():
    table = np.array([[3, -1]])
    _, _, loc, err = oracle.prepare_block(np.zeros(1), np.array([2]), table, 4, 4, 0)
    assert err == ERR_SLOT and loc[0].tolist() == [14, 15, -1, -1]
    _, _, _, err = oracle.prepare_block(np.zeros(1), np.array([5]), table, 4, 4, 0)
    assert err & ERR_CAPACITY
    _, _, loc, err = oracle.prepare_block(np.zeros(1), np.array([0]), np.array([[9, 1]]), 4, 4, 0,
                                          num_pages=5)
    assert err & ERR_SLOT and loc[0, 0] == -1
