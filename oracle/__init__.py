"""CPU oracle of the DSA read path -- test infrastructure, not part of the product.

Only tests/, the package smoke check and the CPU-baseline leg of bench.py may import this
package.  It shares no code with the HIP library or its Python binding.
"""
from .dsa_oracle import *  # noqa: F401,F403
