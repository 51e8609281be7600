"""Float64 CPU oracle for decode-context-parallel (DCP) MLA causal verification.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library or its Python binding, and it never reads the per-rank KV pools that
the GPU reads: it works on the *global* latent sequence and on the ownership
rule stated by the pages.

Sources (the pages this follows):
  * "Context Parallel Guide (PCP & DCP)" (ATOM docs), section
    "Decode Context Parallel (DCP) Guide", the ``interleave_size`` knob,
    "How it works" item 1 (virtual blocks), "DSpark" (local slot / local
    row count) and "enable_project_before_merge" (the merge is a
    per-(token, head) weighting plus a cross-rank sum).
  * "[ROCm][MLA][DCP] Support causal multi-token verification" (vLLM PR
    #51705), "Implementation" items 1-3 and the review thread on
    ``_segmented_mla_page_size``.
  * "[Spec decode] Support Kimi-K3 DCP with DSpark" (vLLM PR #52188), the
    review comment that computes per-query global lengths.

Modules:
  formats    -- decode of BF16 bit patterns and OCP FP8 E4M3 codes to float64
  layout     -- ownership, rank-local token lists, subpage size, metadata and
                KV slots, all by brute-force enumeration of global positions
  attention  -- global causal attention, per-rank split, LSE merges (float64)
  exchange   -- the a2a message layout (LSE as two 16-bit halves) and the
                per-head W_V projection of project-before-merge
  qsplit     -- the exact two-term E4M3 split of BF16 query rows (with a
                round-to-nearest-even E4M3 encoder over the code table)

Every function is pinned by ``tests/test_oracle_*.py`` against what the pages
and mathematics fix (printed examples, closed forms, library routines,
identities).  Nothing here is "parity unpinned".
"""
