"""CPU oracle of the Lighthouse Attention layer.

TEST INFRASTRUCTURE ONLY: a plain, slow, fp64 implementation written from the
two Lighthouse pages (the aitrends.kr summary and the techllm.github.io
review). Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it; the HIP library and its Python binding never do.
"""
from .lighthouse import *  # noqa: F401,F403
from .lighthouse import build_scorer  # noqa: F401
