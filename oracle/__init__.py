"""CPU oracle (test infrastructure only; see tmoe_oracle's module docstring)."""
from .tmoe_oracle import *  # noqa: F401,F403
from . import attention_oracle  # noqa: F401,E402  (the attention half; imported as a module)
