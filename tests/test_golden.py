"""Regression pin of the oracle against its committed greedy run of the tiny
decoder (tests/golden/tiny_greedy.json, written by tests/golden/make_golden.py
from oracle/ alone).  The pages print no worked values for the decode step, so
this pins the oracle to its own committed behaviour; the independent pins are
in test_oracle_pins.py."""

import json
import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


@pytest.fixture(scope="module")
def stored_and_fresh():
    with open(os.path.join(HERE, "golden", "tiny_greedy.json")) as f:
        stored = json.load(f)
    return stored, make_golden.compute()


def test_golden_greedy_tokens(stored_and_fresh):
    stored, fresh = stored_and_fresh
    assert fresh["prompt"] == stored["prompt"]
    assert fresh["greedy_tokens"] == stored["greedy_tokens"]


def test_golden_top_logits(stored_and_fresh):
    stored, fresh = stored_and_fresh
    assert len(fresh["steps"]) == len(stored["steps"])
    for a, b in zip(fresh["steps"], stored["steps"]):
        assert [i for i, _ in a["top"]] == [i for i, _ in b["top"]]
        for (_, va), (_, vb) in zip(a["top"], b["top"]):
            assert abs(va - vb) <= 1e-4 * max(1.0, abs(vb))
        assert abs(a["max_abs"] - b["max_abs"]) <= 1e-4 * max(1.0, b["max_abs"])
