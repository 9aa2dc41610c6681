"""CPU oracle for Block-Union KV Selection and chunked-prefill attention (test infrastructure).

Plain, slow, obviously correct numpy code in float64, written from the CompactAttention pages
("CompactAttention: Accelerating Chunked Prefill with Block-Union KV Selection", abstract):
the per-group KV block tables are the explicit OR of the per-head 2D block masks over the
chunk's Q-blocks and over the query heads of one GQA group, and attention for every query head
of the group runs over exactly the keys of those blocks.

This package is test infrastructure.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code, header, table or constant with the HIP
library, and it imports nothing from it.

Pin status (what each function is checked against besides itself):
  block_union_tables   pinned: brute-force loops, superset/minimality, all-ones/all-zero/G=1
  unpack_mask_bits     pinned: hand-written words (bits 0, 1, 63 of two words) and a per-bit
                       Python-int loop
  paged_attention      pinned: dense causal attention via torch SDPA (all-ones masks),
                       per-token brute force, per-query block-sparse SDPA special case,
                       closed forms (constant V, q=0, single key), LSE-merge identity,
                       page-permutation invariance
  attention_rows       pinned: equals paged_attention on every row it is given
  block_plans          pinned: per-row loop over the definition; G = 1 / one query block equals
                       the union table
  block_sparse_attention / block_sparse_rows
                       pinned: torch SDPA with an explicit per-(head, row) boolean mask over
                       contiguous K/V; equals paged_attention on the union tables when every
                       head of a group shares one mask constant over the query blocks
  decode_e4m3 / dequant_e4m3
                       pinned: code values worked by hand (1, 2, 448, the smallest subnormal,
                       -0, NaN), every code against torch's float8_e4m3fn
  append_kv            pinned: a worked example written out by hand; the appended rows read
                       back through logical positions; every other slot unchanged
"""
from .union import block_union_tables, block_union_tables_bits, unpack_mask_bits  # noqa: F401
from .attention import paged_attention, attention_rows  # noqa: F401
from .append import append_kv  # noqa: F401
from .direct import block_plans, block_sparse_attention, block_sparse_rows  # noqa: F401
from .fp8 import decode_e4m3, dequant_e4m3  # noqa: F401
