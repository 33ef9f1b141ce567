"""Plain, slow, fp64 CPU oracle for blockwise attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library or its Python binding.

Sources (web pages; cited by title and section):

* "Fixed-m softmax for 2D-ring x Ulysses attention (WAN 2.2)" (maxdiffusion
  pull request 452): description, Notes and Tests -- online softmax, the
  per-query Cauchy-Schwarz bound, the per-head gate, the global bound over
  all K shards and the LSE-space merge of hop partials.
* "Let splash attention exceed 524,288 tokens when packing is off" (maxtext
  pull request 4929): description -- segment ids; one segment equals the
  non-segmented kernel.
* sglang pull request 47566 (H3 packed sequence): Motivation and
  Modifications -- cu_seqlens [0, 33002, 33024], alignment rows kept in their
  own segment and zeroed.
* maxdiffusion pull request 404 (ulysses_ring review): padding sits at the end
  of the global sequence; masks come from global positions.
* "Add more optimal dk order optional arg" (flash-attention pull request
  2512): "Sliding window perf issue" -- tiles are partial, full or skipped;
  description -- the backward pass per key column and the order in which
  the key columns add into dQ.

Every function computes the plain definition; none simulates a GPU order of
operations.  Readings of points the pages leave open are listed in the
module docstrings where they are used.
"""

from .attention import (  # noqa: F401
    visibility,
    contiguous,
    kv_head,
    row_intervals_bruteforce,
    row_intervals,
    attention,
    attention_rows,
    fixed_m_safe_max,
    softmax_probs,
    lse_merge,
    fixed_m_bound,
)
from .backward import (  # noqa: F401
    attention_backward,
    attention_backward_heads,
    attention_backward_rows,
    attention_backward_keys,
)
from .blocks import (  # noqa: F401
    FULL,
    PARTIAL,
    SKIP,
    block_kinds_bruteforce,
    block_kinds_intervals,
    runs_from_kinds,
    block_lists,
    counted_flops,
)
