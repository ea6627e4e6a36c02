"""CPU oracle for the GPT-2 training step.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product path.  It shares
no code with the HIP library.  See gpt2_oracle.py for the definitions and the
readings of the source pages they follow.
"""
from .gpt2_oracle import *  # noqa: F401,F403
from .gpt2_oracle import Config, param_specs, num_params, unflatten, decay_mask  # noqa: F401
