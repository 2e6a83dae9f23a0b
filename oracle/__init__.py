"""Independent fp64 CPU oracle for one Wave Forcing wavefront round.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call,
link or execute anything in this package: only ``tests/``, the smoke check in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` use it.
It shares no code with the HIP library (no kernels, headers, helpers, tables
or constants); it imports NumPy and nothing else from this repository.

Source followed throughout ("WF" below): the arXiv HTML page of
"Wave Forcing: Towards Speed-of-Light Streaming Video Generation"
(arXiv 2611.00859).  Each function cites the section / equation it follows.

Modules
-------
wf_plan       schedule, ordered key-page lists, slot ring (integer work)
wf_rope       3D rotary position embedding in fp64
wf_attention  dense softmax attention in fp64
wf_fp8        FP8 (E4M3) page and query quantisation reading
wf_round      one round assembled by logical chunk identity (never by slot)
wf_dit        Wan-shaped DiT block around the round (norms, projections, FFN)

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against printed values, closed forms, invariants or library routines
(torch CPU ``scaled_dot_product_attention``, complex multiplication,
torch's ``float8_e4m3fn``, torch's fp64 norms and GELU, a block composed of
torch modules).
"""
