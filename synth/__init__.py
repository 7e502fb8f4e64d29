"""Seeded synthetic corpora shaped like the workloads the packing pages describe.

This module only draws inputs: token ids, document lengths, source/stratum
labels, prompt lengths and an integer recipe.  It holds none of the packing
arithmetic, so both the CPU oracle and the GPU library can be fed from it.
"""
from .corpus import Corpus, CONFIGS, make_corpus, random_small, recipe_from_shares  # noqa: F401
