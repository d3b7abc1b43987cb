"""CPU oracle (test infrastructure only; see moe_ref)."""
from .moe_ref import *  # noqa: F401,F403
from . import moe_ref  # noqa: F401
