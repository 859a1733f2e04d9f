"""Pins for the whole-word rule (ignore_merges) of the oracle.

TokTier summary page, §4.2: for the Llama family the whole pre-token is first
matched against the vocabulary, and a match skips the merges.  The pages give
no worked example; these pins fix the rule by a hand-worked vocabulary where
it changes the result, and by invariants that any correct implementation
keeps: the text round-trips, a piece never gets more tokens than plain BPE
gives it, pieces that are not vocabulary tokens are encoded exactly as plain
BPE encodes them, and on a vocabulary where every token is its own BPE (as
BPE training produces) the two modes agree everywhere.
"""
import itertools
import os
import random

import numpy as np

from oracle.bpe import Vocab, bpe_classic, decode, encode, encode_offsets
from oracle.pretok import CL100K, GPT2, split_bytes
from synth import code_text, extend_merges, mix_text, word_text

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A, B, C = 97, 98, 99


def test_hand_worked_vocabulary():
    # ab = 256 (rank 0), bc = 257 (rank 1), a + bc = 258 (rank 2).  Plain BPE
    # of "abc" merges the lower-ranked pair ab first and then finds no merge
    # for (ab, c); the vocabulary still holds "abc" as 258.
    v = Vocab([(A, B), (B, C), (A, 257)])
    assert encode(b"abc", v, GPT2) == [256, C]
    assert encode(b"abc", v, GPT2, ignore_merges=True) == [258]
    # "abcc" and "xabc" are no tokens: the same as plain BPE
    assert encode(b"abcc", v, GPT2, ignore_merges=True) == [256, C, C]
    assert encode(b" abc", v, GPT2, ignore_merges=True) == [32, 256, C]
    # one pre-token at a time: " abc abc" splits as " abc" + " abc"? No:
    # GPT-2-style rules give "abc", " abc" for "abc abc"
    assert encode(b"abc abc", v, GPT2, ignore_merges=True) == [258, 32, 256, C]
    # "bc" is reachable by plain BPE too
    assert encode(b"bc", v, GPT2, ignore_merges=True) == [257] == encode(b"bc", v, GPT2)


def test_smallest_id_for_repeated_bytes():
    # "abc" twice in the vocabulary: 257 = ab + c and 259 = a + bc; the rule
    # takes the first id that has those bytes
    v = Vocab([(A, B), (256, C), (B, C), (A, 258)])
    assert v.tok_bytes[257] == v.tok_bytes[259] == b"abc"
    assert encode(b"abc", v, CL100K, ignore_merges=True) == [257]


def test_invariants_on_text():
    base = np.load(os.path.join(ROOT, "data", "vocab_c2.npy"))
    merges = extend_merges(base, 400, 5)
    v = Vocab(merges)
    unreachable = [t for t in range(v.size - 400, v.size) if bpe_classic(v.tok_bytes[t], v.rank) != [t]]
    assert len(unreachable) > 30
    # text with the new tokens as words, plus ordinary code text
    data = word_text(merges, len(base), 600, 6, code_text)
    plain = encode(data, v, GPT2)
    whole = encode(data, v, GPT2, ignore_merges=True)
    assert whole != plain
    assert decode(whole, v).encode() == data
    assert len(whole) < len(plain)
    pieces, _ = split_bytes(data, GPT2)
    for p in set(pieces):
        wp = encode(p, v, GPT2, ignore_merges=True)
        pp = encode(p, v, GPT2)
        assert len(wp) <= len(pp)
        if p in v.token_id:
            assert len(wp) == 1 and v.tok_bytes[wp[0]] == p
        else:
            assert wp == pp
    ids, starts, _ = encode_offsets(data, None, v, GPT2, ignore_merges=True)
    assert ids == whole and starts[-1] == len(data)


def test_trained_vocabulary_modes_agree():
    # every token of a trained table is its own BPE, so the rule changes nothing
    v = Vocab(np.load(os.path.join(ROOT, "data", "vocab_c1.npy")))
    assert all(bpe_classic(v.tok_bytes[t], v.rank) == [t] for t in range(256, v.size))
    for data, pat in ((code_text(20_000, 7), GPT2), (mix_text(20_000, 8, multibyte=True), CL100K)):
        assert encode(data, v, pat, ignore_merges=True) == encode(data, v, pat)


def test_brute_force_short_strings():
    # every string of up to 5 letters over {a, b, c} as one pre-token: one
    # token exactly when it is in the vocabulary, else plain BPE
    v = Vocab([(A, B), (B, C), (A, 257), (256, A), (C, C), (258, 260), (B, B)])
    vocab_strings = set(v.tok_bytes[256:])
    for n in range(1, 6):
        for t in itertools.product(b"abc", repeat=n):
            s = bytes(t)
            got = encode(s, v, GPT2, ignore_merges=True)
            assert decode(got, v).encode() == s
            if s in vocab_strings or n == 1:
                assert len(got) == 1
            else:
                assert got == encode(s, v, GPT2)
