"""Writes thd64k_cu_seqlens_seed4.json: the packed-sequence boundaries the thd64k
workload uses (an input, not an expected value), so a change in the recipe or in
numpy's generator shows up as a test failure."""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import workloads  # noqa: E402

cu = workloads.cu_seqlens_from_lengths(workloads.thd_lengths(4)).tolist()
json.dump({"seed": 4, "total": 65536, "cu_seqlens": cu},
          open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "thd64k_cu_seqlens_seed4.json"), "w"))
