"""CPU oracle of the looped nGPT forward pass (test infrastructure only).

Importable by the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg, nothing else.
"""
from . import sampling
from .model import (LAST_LOOP, PER_LOOP, OracleModel, attend, bf16_round, greedy, l2_normalize,
                    ngpt_residual, rope, self_speculative, self_speculative_reuse, silu)

__all__ = ["sampling", "LAST_LOOP", "PER_LOOP", "OracleModel", "attend", "bf16_round", "greedy", "l2_normalize",
           "ngpt_residual", "rope", "self_speculative", "self_speculative_reuse", "silu"]
