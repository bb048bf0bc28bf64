"""CPU oracle of the Nemotron-H MoE FFN layer forward.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package. The product
path (the HIP library and its Python binding) never imports, calls or links
anything here, and nothing here imports the product package.

Modules:
  moe_oracle  plain float64 NumPy forward of the layer, step by step
  nvfp4       E2M1 / E4M3 decoders and the two-level block quantizer
"""

from . import moe_oracle, nvfp4  # noqa: F401
