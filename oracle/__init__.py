"""The oracle: a plain, slow, CPU-only reference of the PersonaPlex/Moshi temporal
transformer forward and of the 16-position depth transformer that consumes it.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, tables, helpers or
layouts with the HIP library; it computes everything in fp64 with NumPy from the
plain definitions on the pages it cites.

Modules
  temporal   -- embedding sum, RMSNorm, RoPE, windowed causal attention, SwiGLU,
                the 32-block stack (full-sequence and incremental), text head
  depformer  -- the 16-position depth transformer with per-position weights
  inventory  -- tensor shapes and parameter / cache byte arithmetic of the constructor
  ring       -- the integer slot/position arithmetic of a ring KV cache
  sampling   -- temperature / top-k sampling with caller-supplied uniform draws
  generator  -- one generator frame: delayed-code ring, text and depth sampling
  reader     -- memory readers: LayerNorm query, attention over visible memory rows,
                output projection added to the residual

Every function is pinned by tests/test_oracle_*.py against facts the pages fix
(printed counts, integer examples, closed forms, invariants, brute force). The one
part that stays "parity unpinned" is agreement with the released PersonaPlex
checkpoint's numerics: the pages publish no weights or reference outputs.
"""

from . import temporal, depformer, inventory, ring, sampling, generator, reader  # noqa: F401
