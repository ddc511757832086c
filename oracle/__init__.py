"""CPU oracle for the paged KV cache: test infrastructure, not product code.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library: it keeps its
own page store in its own layout ([layer][page][slot][kv_head][dim], the
token-major layout of the AstrAI PagedCache page), addresses tokens with the
block-table rule, quantizes with float32 IEEE operations and computes
attention in float64 after gathering pages into a contiguous copy.

Every function is pinned by a CPU test against something other than itself
(round trips, the page-by-page chunked write, torch's fp64 SDPA on an identity
table, brute-force scalar loops, closed forms, permutation invariance, and
hand-derived pool fixtures).  The int8 rounding rule has no page to compare
against: its parity is pinned by definition and by properties only.
"""
from .paged_cache import OracleCache, quantize_int8_rows, bf16_bits_to_f32  # noqa: F401
from .attention import attend, attend_one, attend_multi, query_positions  # noqa: F401
from .pool import PoolModel, PoolError  # noqa: F401
