"""Float64 CPU oracle (test infrastructure only; see ``lora_oracle``)."""
from .lora_oracle import *  # noqa: F401,F403
