"""Host-side logic of bench.py (no GPU): the near-tie count of a top-p selection."""
import importlib.util
import os

import torch

_spec = importlib.util.spec_from_file_location("bench", os.path.join(os.path.dirname(__file__), "..", "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def test_near_ties_hand_rows():
    # one head, 4 key clusters of which the last is empty; p = 0.8
    A = torch.tensor([[[0.5, 0.3, 0.2, 0.0],      # kept prefix sums exactly to p: a sum near-tie
                       [0.45, 0.45, 0.1, 0.0],    # equal importances at the cut: an order near-tie
                       [0.6, 0.25, 0.15, 0.0],    # prefix 0.85 against 0.6: clear
                       [0.0, 0.0, 0.0, 0.0]]],    # nothing selected: not counted
                     dtype=torch.float32)
    ko = torch.tensor([[0, 1, 2, 3, 3]])
    counts = torch.tensor([[2, 1, 2, 0]])
    r = bench.topp_near_ties(A, ko, counts, 0.8)
    assert r == {"rows": 3, "sum": 1, "order": 1, "tau": 1e-5}


def test_near_ties_p_one():
    A = torch.full((1, 2, 3), 1.0 / 3)
    assert bench.topp_near_ties(A, torch.tensor([[0, 1, 2, 3]]), torch.tensor([[3, 3]]), 1.0)["rows"] == 0
