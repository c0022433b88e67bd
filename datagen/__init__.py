"""Seeded synthetic inputs (shared by the oracle's tests and the HIP path's
tests and bench).  Holds no arithmetic of the MoE layer itself."""
from . import configs
from .configs import ALL, Workload, get
from .gen import generate, random_small, f32_to_bf16_bits
