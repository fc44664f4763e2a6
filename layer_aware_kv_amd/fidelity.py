"""Selection fidelity of the sparse tier, measured on the device.

For a sparse layer that attends over the token set U of the selected pages, the
share of the full-attention probability mass that U captures is

    recall_h = sum_{t in U} softmax(s_h)_t = exp(lse_U,h - lse_full,h),

so it follows from the LSE outputs of the sparse call and of a full-attention call
on the same layer, query and cache.  Together with |out_sparse - out_full| this
shows how closely the selection of a delta-layer (DELTA: top pages by the
per-token maximum attention weight over heads, plus a recency window) serves the
later layers, per layer and over decode steps.
"""
from __future__ import annotations

import torch


def selection_recall(lse_sparse: torch.Tensor, lse_full: torch.Tensor) -> torch.Tensor:
    """Per (row, head) attention mass of the selection under the full softmax."""
    return torch.exp((lse_sparse.float() - lse_full.float()).clamp(max=0.0))


def summarize(recalls: dict, errors: dict) -> dict:
    """recalls / errors: {(step, layer): tensor}; returns plain-number statistics."""
    if not recalls:
        return {}
    allr = torch.cat([r.flatten() for r in recalls.values()])
    steps = sorted({s for s, _ in recalls})
    layers = sorted({l for _, l in recalls})
    q = torch.quantile(allr.double(), torch.tensor([0.05, 0.5], dtype=torch.float64, device=allr.device))
    return {
        "steps": steps,
        "sparse_layers": layers,
        "recall_mean": round(float(allr.mean()), 5),
        "recall_p05": round(float(q[0]), 5),
        "recall_median": round(float(q[1]), 5),
        "recall_min": round(float(allr.min()), 5),
        "per_layer_recall_mean": {str(l): round(float(torch.cat([recalls[(s, l)].flatten() for s in steps
                                                                  if (s, l) in recalls]).mean()), 5)
                                  for l in layers},
        "per_step_recall_mean": {str(s): round(float(torch.cat([recalls[(s, l)].flatten() for l in layers
                                                                 if (s, l) in recalls]).mean()), 5)
                                 for s in steps},
        "max_abs_out_err": round(max(float(e.max()) for e in errors.values()), 5),
        "mean_abs_out_err": round(float(torch.cat([e.flatten() for e in errors.values()]).mean()), 6),
    }
