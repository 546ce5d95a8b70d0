"""CPU oracle for gather_qmm (test infrastructure; never on the product path)."""
from .mq_oracle import *  # noqa: F401,F403
from .mq_oracle import __all__  # noqa: F401
