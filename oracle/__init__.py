"""CPU oracle for the batched paged decode / speculative-verify step.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything in this package. The GPU library never
routes through it and shares no code with it; the two meet only on the
seeded inputs written by ``synth``.

Plain, slow and obviously correct: PyTorch CPU tensor ops in float64, the
library matmul as the only heavy primitive, contiguous per-sequence K/V, no
blocking, fusion or reordering beyond each operation's definition. Every
function cites the page and section it follows.

Modules:
  layers  -- RMSNorm, rotary embedding, standard and key-blockwise
             attention, tile-statistics merge, SiLU / SwiGLU, argmax + gap
  model   -- one decode / verify step over contiguous caches; byte counts
  accept  -- greedy acceptance, expected tokens per pass, rejection-sampling
             distributions
  pool    -- reference model of the refcounted block table with copy-on-write

Parity pins live in tests/test_oracle_*.py. Every function has at least one
pin that does not restate its own formula (printed page values, closed forms,
library routines, invariants, brute force on tiny inputs).
"""
from .accept import accept_greedy, expected_tokens_per_pass, rejection_output_dist  # noqa: F401
from .layers import (argmax_lowest, attention_blockwise, attention_standard, combine_partials,  # noqa: F401
                     linear, rmsnorm, rope, round_to, silu, swiglu)
from .model import SeqState, StepResult, decode_step, kv_bytes_per_token, param_count  # noqa: F401
from .model import streamed_weight_bytes  # noqa: F401
from .pool import PoolModel  # noqa: F401
