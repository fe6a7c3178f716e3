"""fp64 CPU oracle for head-segmented paged prefill attention.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg are the only code that may import or run anything here.
The oracle shares no code with the HIP library (head_segmented_paged_amd).

  tables.py      page-table / segment builder (plain Python)
  attn_fp64.c    fp64 two-pass attention over each head's visible set (C, OpenMP)
  paged.py       the oracle's own paged write + ctypes call of attn_fp64
  bruteforce.py  dense attention with an explicit boolean mask (pin, tiny inputs)
"""
