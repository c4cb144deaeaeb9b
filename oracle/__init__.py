"""Oracle for the integer-only (C, e) training layer step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package.  The
product path (the HIP library and its Python binding) never imports it, and
the oracle never imports the product path: the two share no code.

Everything here follows "Memory-Efficient Integer-Only Training of Deep Neural
Networks" (Shalby, Pittorino, Roveri): the Abstract, Figure 1 (a: forward and
backward of every layer, b: integer-only SGD with momentum and per-group
velocity), Table 5 (per-group velocity / exponent memory), Table 6 (which
primitive each layer uses: product, sum, divide-by-constant) and Table 7 (clip
activations).  The page prints none of the equation bodies it cites, so every
bit-level rule here is a reading; each is named in the function that takes it.
"""

from .ie_oracle import *  # noqa: F401,F403
