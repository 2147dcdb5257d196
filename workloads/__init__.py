"""Workload shapes and seeded synthetic inputs (no arithmetic of the method)."""
from .configs import (BLOCK, PAGE, DrafterConfig, Workload, WORKLOADS, TINY, QWEN3_8B,
                      LLAMA31_8B, GPT_OSS_120B, scaled)
from . import synth
