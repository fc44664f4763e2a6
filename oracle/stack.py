"""One decode step through a layer stack (oracle; test infrastructure only).

"Methodology in Plain English" (DELTA AI summary page): the first two layers
attend to the whole context; a few delta-layers do too and renew the page choice;
the other layers attend to the pages chosen by the most recent delta-layer, a
choice renewed for every generated token.  "Main Findings": the first two layers
are full in every model and the first delta-layer is layer 2.

Readings: a delta-layer's attention output is its full-attention output (the
selection is a side output); a sparse layer that comes before any delta-layer in
the step has no selection and is an error; each layer's new token is appended
before that layer's attention.
"""
from __future__ import annotations

from .attention import full_attention, sparse_attention
from .delta import delta_layer


def layer_tiers(num_layers: int, full_layers, delta_layers) -> list:
    """Tier of every layer: "full", "delta" or "sparse"."""
    tiers = []
    for layer in range(num_layers):
        if layer in full_layers:
            tiers.append("full")
        elif layer in delta_layers:
            tiers.append("delta")
        else:
            tiers.append("sparse")
    return tiers


def stack_step(tiers, layer_inputs, sm_scale: float, page: int, k_top: int, recency: int,
               agg: str = "max", scope: str = "group"):
    """One decode step of one sequence through the stack.

    ``layer_inputs[l]`` = (q [Hq, D], K [Hkv, T, D], V [Hkv, T, D]) of layer l with
    this step's token already appended.  Returns a list of per-layer dicts with
    ``out``, ``lse`` and, for delta-layers, ``sel``; sparse layers record the
    selection they used under ``sel_used``.
    """
    results = []
    sel = None
    for layer, tier in enumerate(tiers):
        q, K, V = layer_inputs[layer]
        if tier == "full":
            out, lse, _ = full_attention(q, K, V, sm_scale)
            results.append(dict(out=out, lse=lse))
        elif tier == "delta":
            r = delta_layer(q, K, V, sm_scale, page, k_top, recency, agg, scope)
            sel = r["sel"] if scope == "group" else r["sel"][0]
            results.append(dict(out=r["out"], lse=r["lse"], sel=r["sel"], page_scores=r["page_scores"]))
        else:
            if sel is None:
                raise ValueError(f"sparse layer {layer} has no preceding delta-layer")
            out, lse = sparse_attention(q, K, V, sel, page, sm_scale)
            results.append(dict(out=out, lse=lse, sel_used=sel))
    return results
