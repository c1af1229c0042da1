"""fp64 CPU oracle for the tiled attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and this package
imports nothing from the product path; the two share only the seeded input
generators in ``attn_workloads``.

Contents
--------
materialised  materialised scores + exact softmax, the plain definition of
            scaled-dot-product attention (page "gfx942 unified attention, from
            the math up", sections 1, 2, 4, 5), with the bottom-right causal
            mask, paged-KV gather and the GQA head map.
online      a brute-force online-softmax (streaming) evaluation of the same
            quantity with an arbitrary tile width (same page, section 3), used
            only as a checker of ``attention``.
combine     the log-sum-exp merge of split-KV partial results (same page,
            section 8: partial softmax-weighted outputs combined), plus the
            per-split partials themselves.
brute       pure-Python per-row evaluation for tiny inputs (math.exp/fsum).
rounding    rounding to bfloat16 with ties to even, ties away from zero, or toward
            zero (the three output modes of the MoonMath benchmark page).

Parity pins: every function above is pinned by ``tests/test_oracle.py`` against
closed forms, invariants, a library special case (torch CPU SDPA in float64)
and hand-derived golden fixtures; none is "parity unpinned".
"""
from .materialised import attention, attention_rows, gather_kv, kv_head_of  # noqa: F401
from .online import online_attention_rows  # noqa: F401
from .combine import lse_combine, split_partials  # noqa: F401
from .rounding import round_bf16  # noqa: F401
