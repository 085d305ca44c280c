"""CPU oracle of the contextual-sparsity LoRA hot path (test infrastructure).

Imported only by the tests, the smoke check and the benchmark's CPU
baseline; the product library never loads anything from here.
"""
from .sparselora_oracle import *  # noqa: F401,F403
from .sparselora_oracle import __all__ as _core_all
from .quant4 import *  # noqa: F401,F403
from .quant4 import __all__ as _quant_all

__all__ = list(_core_all) + list(_quant_all)
