"""CPU oracle for MoE dispatch/combine — test infrastructure, not product.

Only the tests, the smoke entry and the benchmark's cpu_baseline leg may
import this package.  See ``oracle.ep_oracle`` for the definitions.
"""
from .ep_oracle import *  # noqa: F401,F403
from .ep_oracle import __all__  # noqa: F401
