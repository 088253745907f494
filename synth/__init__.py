"""Seeded synthetic inputs shared by the CPU oracle and the GPU path."""
from .inputs import *  # noqa: F401,F403
from .inputs import CONFIGS, LayerConfig, LayerWeights, W4  # noqa: F401
