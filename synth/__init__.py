"""Seeded synthetic workloads (texts and training corpora).

This package only draws text: it holds none of the tokenization arithmetic and
is the one module that both the oracle-side tests and the GPU-side tests and
benchmark import for their inputs.
"""
from .text import (  # noqa: F401
    ASCII_PUNCT,
    lexicon,
    code_text,
    mix_text,
    batch_texts,
    adversarial_text,
    random_word,
    workload,
    WORKLOADS,
)
from .vocab import extend_merges, word_text  # noqa: F401
