"""Host-side helpers of bench.py (no GPU): the routing load-balance fields and
the sampled parity record of the bench line, on small hand-made cases."""
import os
import sys
from types import SimpleNamespace

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_routing_stats_by_hand():
    s = bench.routing_stats([0, 1, 1, 6])
    assert s["empty_experts"] == 1 and s["one_row_experts"] == 2 and s["max_group_rows"] == 6
    # mean 2, population std sqrt((4 + 1 + 1 + 16) / 4)
    assert abs(s["load_std_over_mean"] - round(np.sqrt(22 / 4) / 2, 4)) < 1e-12
    assert bench.routing_stats([0, 0])["load_std_over_mean"] is None
    assert bench.routing_stats([5, 5, 5])["load_std_over_mean"] == 0.0


def test_sampled_parity_skips_rerouted_tokens():
    ref_out = np.array([[1.0, -2.0], [0.5, 0.25], [3.0, 3.0]], dtype=np.float32)
    ref = SimpleNamespace(out=ref_out, topk_idx=np.array([[0, 1], [2, 3], [1, 0]], dtype=np.int32))
    gpu = torch.tensor(ref_out).to(torch.bfloat16)
    gpu = torch.cat([gpu, torch.zeros((1, 2), dtype=torch.bfloat16)])   # one token past the sample
    gpu[0, 1] = -2.0625                                                # |err| 1/16 on a max of 2
    gpu[2, 0] = 100.0                                                  # a token routed elsewhere
    idx = torch.tensor([[0, 1], [2, 3], [1, 2], [4, 5]], dtype=torch.int32)
    p = bench.sampled_parity(gpu, idx, ref)
    assert p["tokens"] == 3 and p["routing_differs"] == 1
    assert abs(p["max_token_rel_err"] - 0.0625 / 2) < 1e-7


def test_source_hash_ignores_comments_only():
    """Stored counter data stays valid across comment edits, not code edits."""
    a = bench._code_only("int f(int x) {  // twice\n  return 2 * x; /* doubled */\n}\n")
    b = bench._code_only("int f(int x) {\n  return 2 * x;\n}")
    c = bench._code_only("int f(int x) {\n  return 3 * x;\n}")
    assert a == b and a != c
