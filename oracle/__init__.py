"""CPU oracle for DELTA's decode-time attention hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package;
the library under ``layer_aware_kv_amd/`` never does, and shares no code with it.

Source of the definitions: "DELTA: Dynamic Layer-Aware Token Attention for
Efficient Long-Context Reasoning", AI summary page, sections "Methodology in
Plain English" (three layer tiers; a delta-layer attends to the whole context,
scores each token by its largest softmax weight over the heads, scores each
page of 16 tokens by adding its tokens' scores, and chooses a window of the
newest pages plus, up to the budget, the older pages of largest score; the
other layers attend to the chosen pages only; the choice is renewed at every
delta-layer and for every generated token; no token leaves the KV cache) and
"Main Findings" (budget of K pages plus a window of L recent pages; the first
two layers attend fully and the first delta-layer is layer 2).

Everything is plain NumPy in float64, one (batch row, head) at a time, in the
order the pages state the steps.  Readings of points the pages leave open are
listed in each function's docstring.

fp8 KV pages (``quant``): OCP E4M3 codes with one float32 scale per (token,
KV head) row; the pages name quantization as a technique to combine with DELTA
("Future Directions") and fix no format, so the format and its readings are
stated in that module.

Pins (tests/test_oracle_*.py): torch's scaled_dot_product_attention in float64,
scipy's logsumexp, torch's float8_e4m3fn conversions, closed forms, brute-force
subset search for the selection, and the invariants the pages state (no
eviction; all delta-layers -> full attention).  Parity status of every function:
pinned.
"""
from .attention import full_attention, sparse_attention, attention_over_tokens  # noqa: F401
from .delta import token_scores, page_scores, select_pages, delta_layer  # noqa: F401
from .stack import layer_tiers, stack_step  # noqa: F401
from . import quant  # noqa: F401
