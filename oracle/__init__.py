"""CPU oracle for DELTA's decode-time attention hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package;
the library under ``layer_aware_kv_amd/`` never does, and shares no code with it.

Source of the definitions: "DELTA: Dynamic Layer-Aware Token Attention for
Efficient Long-Context Reasoning", AI summary page, sections "Methodology in
Plain English" (three layer tiers; delta-layers run full attention, take the
per-token maximum attention weight across heads, group tokens into fixed-size
pages, sum the per-token scores in a page, keep the most recent pages and fill
the rest of the budget with the highest-scoring older pages; sparse layers
attend only to the selected pages; selections refreshed at each delta-layer and
for every generated token; full KV cache kept; page size 16) and "Main Findings"
(budget K pages plus a recency window of L pages; layers 0 and 1 full, layer 2
the first delta-layer).

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
