"""CPU oracle of the Lighthouse attention layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path (HIP library and binding) never does. It shares no code
with the HIP path and imports nothing from it.
"""

from .lighthouse import *  # noqa: F401,F403
from .lighthouse import Config, REFINE, DIRECT, SCORERS  # noqa: F401
