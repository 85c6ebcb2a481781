"""CPU oracle for load-balanced paged decode attention.  TEST INFRASTRUCTURE.

This package is a plain, slow, obviously correct NumPy (fp64) statement of
what the hot path computes.  It exists only to check the HIP library: it may
be imported by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``, and by nothing else.  It shares no code
with the HIP path and imports nothing from it.

Sources (the pages the method is described on):

* SGLang x HPC-Ops page ("HPC-Ops integrated into SGLang", news.ainew.jp),
  sections "Attention: load balancing for mixed-length decode" and
  "Scheduling around live KV work".
* vLLM x HPC-Ops page ("vLLM x HPC-Ops: High-Performance Attention and MoE
  Backends from Tencent Hunyuan"), section "Solution: per-step
  load-balanced decode scheduler", bullets "Assign" and "Compute and
  combine", plus the static split-KV description under "Challenge".

Modules:

* ``assign``    - task maps: the dynamic (budgeted, head-major) assigner and
                  the two static split-KV policies.
* ``attention`` - fp64 paged GQA decode attention, per-range partials with
                  log-sum-exp, and the LSE combine.
* ``e4m3``      - OCP FP8 e4m3 decoding table.

Every function is pinned by CPU tests against hand-worked examples,
brute force on tiny inputs, closed forms, invariants and library routines;
none is marked "parity unpinned".
"""

from . import assign, attention, e4m3, prologue  # noqa: F401
