"""CPU oracle for GPTQ layer-wise quantization (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the product path never imports it.
"""
from .gptq_oracle import *  # noqa: F401,F403
from .gptq_oracle import storage_bits_per_weight, n_groups_total  # noqa: F401
