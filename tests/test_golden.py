"""The oracle reproduces its frozen trajectory, and the pages' printed facts."""
import json
import os

import numpy as np

import workloads

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_trajectory_frozen(oracle_mod):
    with open(os.path.join(GOLD, "e4_trajectory_64.json")) as f:
        gold = json.load(f)
    h = gold["hyper"]
    p = workloads.host_params(1, limit=64)[0]
    w = np.zeros(64, np.uint32)
    for rec in gold["steps"]:
        t = rec["step"]
        g = workloads.host_grads(1, t, limit=64)[0]
        s = oracle_mod.scalars(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], t)
        oracle_mod.step_packed(oracle_mod.PACKED_E4, p, g, w, s)
        assert [f"{x:08x}" for x in p.view(np.uint32)] == rec["params_hex"]
        assert [f"{x:08x}" for x in w] == rec["words_hex"]


def test_oracle_block_length_is_the_pages(oracle_mod):
    with open(os.path.join(GOLD, "pages_facts.json")) as f:
        facts = json.load(f)
    assert oracle_mod.BLOCK == facts["blockwise"]["block"]
    assert oracle_mod._load().oracle_block_len() == facts["blockwise"]["block"]
    qm, qv = workloads.code_maps()
    assert qm.size == qv.size == facts["blockwise"]["map_entries"]
