"""CPU oracle for exact byte-level BPE tokenization -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct definition of what the GPU
path must compute.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product library
(``exact_byte_level_amd``) never imports, links or executes anything here, and
this package never imports the product library: the two share no code.

What it follows (TokTier, arXiv:2607.29678v1, summary page):
  * the pipeline factorisation F = E* o G of Appendix A.1: G splits the text
    into pre-tokens with a sequential regex, E runs BPE on each pre-token with
    no state crossing pre-tokens, and the output is the concatenation;
  * §1.2 / §3.2: exactness is the contract (token ids equal to the reference
    tokenizer's); the tokenizer is not concatenative (tok(A)+tok(B) may differ
    from tok(A+B)).

Modules
  pretok  -- the ordered rule sets and split(); split_bytes() (byte offsets of
             the pieces of one text) and piece_starts_batch() (a batch of
             independent texts)
  bpe     -- the merge-table container Vocab, the classic lowest-rank-first
             merge loop, a heap/linked-list form with the same semantics, the
             naive rank-order brute force, encode / encode_batch, decode, and
             the byte offset of every token
  train   -- the BPE trainer that learns merge tables from seeded corpora

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(worked examples, brute force against independent formulations, closed forms,
invariants, and a third-party implementation where one is installed).  Equality
with the real GPT-2 / cl100k vocabularies is parity unpinned: their pattern
strings and vocab files are not available here.
"""
