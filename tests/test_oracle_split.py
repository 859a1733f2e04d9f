"""Pins for the oracle pre-tokenizer (oracle.pretok).

What pins it, besides itself:
  * worked examples derived by hand from the two rule tables;
  * a second formulation (tests/runsplit.py: the run-decomposition predicate of
    TokTier summary page §4.1, evaluated without any regex engine) that must
    agree on every string of length <= 5 over a class-covering alphabet and on
    random longer strings;
  * a third-party implementation: HF ``tokenizers``' built-in GPT-2 ByteLevel
    pre-tokenizer (its own copy of the GPT-2 pattern, run by Oniguruma), and the
    cl100k-style pattern string run by Oniguruma instead of ``regex``;
  * the whitespace set equals the ``regex`` module's \\s (Unicode White_Space).
"""
import itertools
import random
import re

import pytest
import regex

from oracle.pretok import (CL100K, DEEPSEEK, GPT2, O200K, PATTERNS, WHITESPACE_CPS, _DEEPSEEK_STAGES,
                           piece_starts_batch, split, split_bytes)
from runsplit import piece_starts

EXAMPLES = [
    # (text, GPT-2-style pieces, cl100k-style pieces)
    ("don't", ["don", "'t"], ["don", "'t"]),
    ("DON'T", ["DON", "'", "T"], ["DON", "'T"]),
    ("a  b", ["a", " ", " b"], ["a", " ", " b"]),
    ("12345", ["12345"], ["123", "45"]),
    (" 123", [" 123"], [" ", "123"]),
    ("x'ya", ["x", "'", "ya"], ["x", "'ya"]),
    ("\n\nfoo", ["\n", "\n", "foo"], ["\n\n", "foo"]),
    (";\n\n  foo", [";", "\n\n ", " foo"], [";\n\n", " ", " foo"]),
    (".\tfoo", [".", "\t", "foo"], [".", "\tfoo"]),
    (" .foo", [" .", "foo"], [" .", "foo"]),
    ("x.'s", ["x", ".'", "s"], ["x", ".'", "s"]),
    ("it's", ["it", "'s"], ["it", "'s"]),
    ("'stop", ["'s", "top"], ["'s", "top"]),
    ("we'll go", ["we", "'ll", " go"], ["we", "'ll", " go"]),
    ("x 's", ["x", " '", "s"], ["x", " '", "s"]),
    ("a   ", ["a", "   "], ["a", "   "]),
    ("a \n b", ["a", " \n", " b"], ["a", " \n", " b"]),
    ("a\n \n  b", ["a", "\n \n ", " b"], ["a", "\n \n", " ", " b"]),
    ("1234567", ["1234567"], ["123", "456", "7"]),
    ("x+=1", ["x", "+=", "1"], ["x", "+=", "1"]),
    ("foo_bar", ["foo", "_", "bar"], ["foo", "_bar"]),
    ("中文 é", ["中文", " é"], ["中文", " é"]),
    ("a\r\nb", ["a", "\r", "\n", "b"], ["a", "\r\n", "b"]),
]


@pytest.mark.parametrize("text,gpt2,cl100k", EXAMPLES)
def test_worked_examples(text, gpt2, cl100k):
    assert split(text, GPT2) == gpt2
    assert split(text, CL100K) == cl100k


# o200k-style, worked by hand from its rule table (Q1..Q7):
EXAMPLES_O200K = [
    ("HelloWorld", ["Hello", "World"]),        # Q1 ends at the upper-case W after lower-case o
    ("HTMLParser", ["HTMLParser"]),            # upper-type run, then the lower-type run
    ("aBcD", ["a", "Bc", "D"]),                # D: no lower-case char after it, Q2
    ("ABªCD", ["ABª", "CD"]),                  # lower-type run takes only the last Lo char
    ("don't stop", ["don't", " stop"]),        # the contraction stays with its word
    ("AB'S", ["AB'S"]),                        # Q2 + contraction, case-insensitive
    ("it'sªBc", ["it's", "ªBc"]),              # a word restarts after the contraction
    ("a's's", ["a's", "'s"]),                  # no word ends at the second apostrophe
    ("a's's's", ["a's", "'s's"]),              # ... so attachment alternates
    ("a/\n/b", ["a", "/\n/", "b"]),            # Q4: "other" run, then CR/LF and '/'
    (".\n/.b", [".\n/", ".b"]),                # the tail ends; '.' leads the next word
    ("..\u0301a", ["..", "\u0301a"]),          # marks are letter-type, not "other"
    (" 12345", [" ", "123", "45"]),
    ("x\n \n  y", ["x", "\n \n", " ", " y"]),
    ("\u00c9t\u00e9 2024!\n", ["\u00c9t\u00e9", " ", "202", "4", "!\n"]),
]


@pytest.mark.parametrize("text,pieces", EXAMPLES_O200K)
def test_worked_examples_o200k(text, pieces):
    assert split(text, O200K) == pieces


# DeepSeek-style, worked by hand from its three splits (S1 digits, S2 CJK and
# kana runs, S3 rules D1..D6 on every piece by itself):
EXAMPLES_DEEPSEEK = [
    ("Hello world", ["Hello", " world"]),      # D2 with a leading space
    (".abc\u00e9", [".abc", "\u00e9"]),          # D1 takes ASCII letters only
    ("_foo_bar", ["_foo", "_bar"]),            # '_' is ASCII punctuation: D1 twice
    ("\u20acfoo", ["\u20ac", "foo"]),            # a non-ASCII symbol is a D3 run
    ("x1234567y", ["x", "123", "456", "7", "y"]),
    ("\u4e2d\u6587abc", ["\u4e2d\u6587", "abc"]),   # S2 cuts the CJK run out
    ("\u3042\u30fb\u3044", ["\u3042", "\u30fb", "\u3044"]),  # S3 splits inside a kana run
    (" .a", [" .", "a"]),                      # D3 takes the space; 'a' stands alone
    ("\t.a", ["\t", ".a"]),
    ("a\x00\x01b", ["a", "\x00", "\x01b"]),     # no rule takes \x00; \x01 leads a word
    ("foo()\n\n  bar", ["foo", "()\n\n", " ", " bar"]),
    ("a  1", ["a", "  ", "1"]),                # the segment ends at the digit
    ("don't", ["don", "'t"]),
]


@pytest.mark.parametrize("text,pieces", EXAMPLES_DEEPSEEK)
def test_worked_examples_deepseek(text, pieces):
    assert split(text, DEEPSEEK) == pieces


def _starts(pieces):
    out, pos = [], 0
    for p in pieces:
        out.append(pos)
        pos += len(p)
    return out


ALPHA = ["a", "s", "r", "e", "S", "1", ".", "'", " ", "\n", "\t", "\r"]


@pytest.mark.parametrize("pattern_id", [GPT2, CL100K])
def test_exhaustive_short_strings_against_run_decomposition(pattern_id):
    bad = []
    for length in range(6):
        for tup in itertools.product(ALPHA, repeat=length):
            s = "".join(tup)
            if _starts(split(s, pattern_id)) != piece_starts(s, pattern_id):
                bad.append(s)
    assert bad == []


ALPHA2 = ALPHA + list("lLvVmdDtTEé中😀") + ["　", "\xa0", "2", "²", "_", "(", "\x0b", "٣"]

# o200k-style: both cases, an Lo letter, a combining mark, '/', contractions
ALPHA_O = ["a", "A", "s", "S", "r", "e", "\u00aa", "\u0301", "1", ".", "/", "'", " ", "\n"]
ALPHA_O2 = ALPHA2 + ["\u00aa", "\u0301", "\u01c5", "\u02b0", "/", "\u00c9", "\u0915\u093f"]


def test_exhaustive_short_strings_o200k():
    bad = []
    for length in range(6):
        for tup in itertools.product(ALPHA_O, repeat=length):
            s = "".join(tup)
            if _starts(split(s, O200K)) != piece_starts(s, O200K):
                bad.append(s)
    assert bad == []


ALPHA_D = ["a", "A", "\u00e9", "\u0301", "1", "\u4e2d", "\u3042", "\u30fb", ".", "_", "\u20ac", " ", "\t", "\n",
           "\x00"]
ALPHA_D2 = ALPHA_D + list("sSzZ09$'(") + ["\u6587", "\u309b", "\u30fc", "\u30a2", "\u30a0", "\u00b2", "\u0663", "\r",
                                        "\xa0", "\u200b", "\ue000", "\U0001f600", "\u01c5"]


def test_exhaustive_short_strings_deepseek():
    bad = []
    for length in range(5):
        for tup in itertools.product(ALPHA_D, repeat=length):
            s = "".join(tup)
            if _starts(split(s, DEEPSEEK)) != piece_starts(s, DEEPSEEK):
                bad.append(s)
    assert bad == []


def test_random_strings_deepseek():
    rng = random.Random(19)
    for _ in range(30_000):
        s = "".join(rng.choice(ALPHA_D2) for _ in range(rng.randint(6, 30)))
        assert _starts(split(s, DEEPSEEK)) == piece_starts(s, DEEPSEEK), repr(s)


def test_random_strings_o200k():
    rng = random.Random(17)
    for _ in range(30_000):
        s = "".join(rng.choice(ALPHA_O2) for _ in range(rng.randint(6, 30)))
        assert _starts(split(s, O200K)) == piece_starts(s, O200K), repr(s)


@pytest.mark.parametrize("pattern_id", [GPT2, CL100K])
def test_random_strings_against_run_decomposition(pattern_id):
    rng = random.Random(11 + pattern_id)
    for _ in range(30_000):
        s = "".join(rng.choice(ALPHA2) for _ in range(rng.randint(6, 30)))
        assert _starts(split(s, pattern_id)) == piece_starts(s, pattern_id), repr(s)


def test_long_runs_against_run_decomposition():
    texts = ["a" + "1" * 1000 + "x", ".\n" * 3 + "\n" * 500 + " " * 700 + "z", " " * 999 + "7",
             "\t" * 5 + "\n" + " " * 400, "x" + "٣" * 11 + "2" * 7]
    for t in texts:
        for pat in (GPT2, CL100K, O200K, DEEPSEEK):
            assert _starts(split(t, pat)) == piece_starts(t, pat)


# Characters both engines classify identically (no U+001C..001F, no recent code points).
HF_ALPHA = ALPHA + list("lLvVmdDtTEé中xyz09_(){};:,") + ["\xa0", "　", "é"]


def test_gpt2_split_matches_hf_bytelevel():
    pre = pytest.importorskip("tokenizers.pre_tokenizers")
    bl = pre.ByteLevel(add_prefix_space=False, use_regex=True)
    rng = random.Random(5)
    for _ in range(5000):
        s = "".join(rng.choice(HF_ALPHA) for _ in range(rng.randint(1, 40)))
        hf = [a for _, (a, _) in bl.pre_tokenize_str(s)]
        assert _starts(split(s, GPT2)) == hf, repr(s)


def test_cl100k_pattern_under_oniguruma_matches_regex_module():
    tk = pytest.importorskip("tokenizers")
    # Oniguruma reads a two-digit hex escape as a raw byte; spell code points as x{...}.
    pat = re.sub(r"\\(?:x([0-9a-f]{2})|u([0-9a-f]{4}))", lambda m: "\\x{%s}" % (m.group(1) or m.group(2)),
                 PATTERNS[CL100K])
    sp = tk.pre_tokenizers.Split(tk.Regex(pat), behavior="isolated")
    rng = random.Random(6)
    for _ in range(5000):
        s = "".join(rng.choice(HF_ALPHA) for _ in range(rng.randint(1, 40)))
        hf = [a for _, (a, _) in sp.pre_tokenize_str(s)]
        assert _starts(split(s, CL100K)) == hf, repr(s)


def test_o200k_pattern_under_oniguruma_matches_regex_module():
    tk = pytest.importorskip("tokenizers")
    pat = re.sub(r"\\(?:x([0-9a-f]{2})|u([0-9a-f]{4}))", lambda m: "\\x{%s}" % (m.group(1) or m.group(2)),
                 PATTERNS[O200K])
    sp = tk.pre_tokenizers.Split(tk.Regex(pat), behavior="isolated")
    rng = random.Random(7)
    alpha = HF_ALPHA + ["\u00aa", "\u0301", "/", "\u00c9", "'", "S", "R", "E"]
    for _ in range(5000):
        s = "".join(rng.choice(alpha) for _ in range(rng.randint(1, 40)))
        hf = [a for _, (a, _) in sp.pre_tokenize_str(s)]
        assert _starts(split(s, O200K)) == hf, repr(s)


def test_deepseek_splits_under_oniguruma_match_regex_module():
    tk = pytest.importorskip("tokenizers")

    def onig(p):
        return re.sub(r"\\(?:x([0-9a-f]{2})|u([0-9a-f]{4}))", lambda m: "\\x{%s}" % (m.group(1) or m.group(2)), p)
    seq = tk.pre_tokenizers.Sequence([tk.pre_tokenizers.Split(tk.Regex(onig(p)), behavior="isolated")
                                      for p in _DEEPSEEK_STAGES])
    rng = random.Random(8)
    alpha = HF_ALPHA + ["\u3042", "\u30fb", "\u20ac", "$", "\x01"]
    for _ in range(5000):
        s = "".join(rng.choice(alpha) for _ in range(rng.randint(1, 40)))
        hf = [a for _, (a, _) in seq.pre_tokenize_str(s)]
        assert _starts(split(s, DEEPSEEK)) == hf, repr(s)


def test_whitespace_set_is_unicode_white_space():
    s = regex.compile(r"\s")
    got = [cp for cp in range(0x110000) if not 0xD800 <= cp <= 0xDFFF and s.match(chr(cp))]
    assert got == sorted(WHITESPACE_CPS)
    assert len(WHITESPACE_CPS) == 25
    # str.isspace disagrees on the four information separators; we follow \s.
    assert all(chr(c).isspace() for c in range(0x1C, 0x20))
    assert not any(c in WHITESPACE_CPS for c in range(0x1C, 0x20))


def test_split_bytes_offsets_and_invalid_utf8():
    data = "x é中 12".encode()
    pieces, starts = split_bytes(data, CL100K)
    assert b"".join(pieces) == data
    assert starts == [0, 1, 7, 8]
    for bad in (b"\xff", b"a\x80", b"\xc3", b"\xed\xa0\x80", b"\xc0\xaf", b"\xf4\x90\x80\x80"):
        with pytest.raises(UnicodeDecodeError):
            split_bytes(bad, GPT2)


# A batch is a list of independent fresh texts (TokTier summary page, Appendix
# A.1: the pipeline runs per text; the batch workload's texts are fresh
# sessions), so piece starts restart at every text and no piece crosses a text
# end.  Expected starts written by hand, as byte offsets into the
# concatenation; each text's reading:
#   0  "ab "   -> "ab" | " "      (the space ends its text: the lookahead rule
#                                  sees end-of-text; run on into text 2 it
#                                  would have joined "cd" as " cd")
#   1  ""      -> nothing
#   2  "cd"    -> "cd"
#   3  "é1"    -> "é" (2 bytes) | "1"
#   4  "  x"   -> " " | " x"
#   5  "中 "   -> "中" (3 bytes) | " "
#   6  "1234"  -> GPT-2-style one digit run; cl100k-style "123" | "4"
BATCH_TEXTS = ["ab ", "", "cd", "é1", "  x", "中 ", "1234"]
BATCH_STARTS = {
    GPT2: [0, 2, 3, 5, 7, 8, 9, 11, 14, 15],
    CL100K: [0, 2, 3, 5, 7, 8, 9, 11, 14, 15, 18],
    O200K: [0, 2, 3, 5, 7, 8, 9, 11, 14, 15, 18],  # as cl100k-style: no case or tail rule applies
    DEEPSEEK: [0, 2, 3, 5, 7, 8, 9, 11, 14, 15, 18],  # "中" is its own run piece either way
}


def _batch(texts):
    data, offs = b"", [0]
    for t in texts:
        data += t.encode()
        offs.append(len(data))
    return data, offs


@pytest.mark.parametrize("pattern_id", [GPT2, CL100K, O200K, DEEPSEEK])
def test_piece_starts_batch_hand_worked(pattern_id):
    data, offs = _batch(BATCH_TEXTS)
    assert offs == [0, 3, 3, 5, 8, 11, 15, 19]
    assert piece_starts_batch(data, offs, pattern_id) == BATCH_STARTS[pattern_id]
    # the same bytes split as one text: the space of text 0 joins "cd", so no
    # piece starts at byte 3
    whole = _starts(split(data.decode(), pattern_id))
    assert 3 not in [len(data.decode()[:i].encode()) for i in whole]


@pytest.mark.parametrize("pattern_id", [GPT2, CL100K, O200K, DEEPSEEK])
def test_piece_starts_batch_random_against_run_decomposition(pattern_id):
    """Random batches (empty texts, texts ending in whitespace, multibyte chars)
    against the regex-free run decomposition, applied text by text and shifted
    by each text's byte offset."""
    rng = random.Random(31 + pattern_id)
    for _ in range(400):
        texts = ["".join(rng.choice(ALPHA2) for _ in range(rng.choice([0, 0, 1, 3, 9, 25])))
                 for _ in range(rng.randint(1, 8))]
        data, offs = _batch(texts)
        want = []
        for s, t in enumerate(texts):
            for ci in piece_starts(t, pattern_id):
                want.append(offs[s] + len(t[:ci].encode()))
        assert piece_starts_batch(data, offs, pattern_id) == want, texts
