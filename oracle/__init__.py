"""CPU oracle (test infrastructure only; see tmoe_oracle's module docstring)."""
from .tmoe_oracle import *  # noqa: F401,F403
