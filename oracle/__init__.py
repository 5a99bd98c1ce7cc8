"""CPU oracle for the token-choice sparse MoE FFN forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this package.  The product path (the
HIP library and its Python binding) never imports, calls or links anything
here, and this package imports nothing from the product path: the two share no
code.  Inputs reach both sides from the seeded generator, which holds none of
the method's arithmetic.

Everything is plain NumPy in float64, written from the method's definition on
the source pages; each function cites the passage it follows.  Parity status of
every function is listed in ``moe_oracle.PARITY_PINS``.
"""

from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
