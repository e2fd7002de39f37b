"""The seeded input recipes are stable (CPU only)."""
import json
import os

import numpy as np

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_thd_length_mix_recipe():
    for seed in range(6):
        lens = workloads.thd_lengths(seed)
        assert sum(lens) == 65536
        assert all(x % 8 == 0 for x in lens)
        assert all(128 <= x <= 16384 for x in lens[:-1])
        cu = workloads.cu_seqlens_from_lengths(lens)
        assert cu[0] == 0 and cu[-1] == 65536 and np.all(np.diff(cu) > 0)


def test_thd_fixture_reproduces():
    fx = json.load(open(os.path.join(GOLDEN, "thd64k_cu_seqlens_seed4.json")))
    assert workloads.cu_seqlens_from_lengths(workloads.thd_lengths(fx["seed"])).tolist() == fx["cu_seqlens"]


def test_randn_is_seeded_and_bf16_exact():
    a = workloads.randn((4, 2, 8), 3, "bf16", 1)
    b = workloads.randn((4, 2, 8), 3, "bf16", 1)
    c = workloads.randn((4, 2, 8), 3, "bf16", 2)
    assert (a.float() == b.float()).all() and not (a.float() == c.float()).all()
    assert (a.float().to(a.dtype).float() == a.float()).all()
