"""CPU oracle for budgeted KV-cache compaction.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (``budgeted_retention_amd``) and imports nothing from it.

Everything here is plain numpy in float64, written to be read against the
three pages it follows:

* PASK -- "Parser Transitions Already Reveal Structural Responsibility: KV
  Persistence for Structured Generation".
* PACE -- "PACE: Keeping the Right Tokens in the KV Cache Is Not Enough for
  Long-Horizon LLM Agents".
* CommitKV -- "CommitKV: Lifecycle-Aware KV Cache Compression via Commit
  Transitions for Multi-Turn Agents".

bf16 tensors enter as their raw uint16 bit patterns and are widened exactly
to float64; outputs that the library produces in bf16 are rounded once,
round-to-nearest-even, from the float64 result.

Modules:

* ``numfmt``      -- exact bf16/fp16 <-> float64 conversions.
* ``rope``        -- split-half rotary rotation R_p (PACE §2, Eq. 1).
* ``score``       -- observation-window attention score.
* ``policy``      -- layer groups, foresight bonus, bonus/floor table.
* ``select``      -- top-B selection under the budget.
* ``compact``     -- gather, renumber and exact re-rotation.
* ``quant``       -- symmetric per-token-per-head int8 codes.
* ``decode``      -- decode attention over the compacted cache.
* ``page_effect`` -- CommitKV deletion effects, lifecycle labels, greedy test.
* ``pask``        -- PASK online structural control (Alg. 2).

Parity status: every function has pins in ``tests/test_oracle_*.py`` except
where its docstring says "parity unpinned".
"""
