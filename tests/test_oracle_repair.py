"""Pins for the splice rule of incremental repair, checked on the oracle.

Incremental repair (TokTier summary page, §3.3; splicing theorem, Appendix
A.2) encodes only a window W = X[w0:] of the new text X = A + D and keeps the
old text A's pre-tokens before a splice point p.  The library takes as p a
pre-token start of W with
  * at least 4 chars of W before it and at least 5 chars of A after it (the
    library states these margins in bytes: 16 and 20), and
  * for cl100k-style rules, a change of char class (letter / number /
    whitespace / other) between p - 1 and p.
The claim is that X's pre-token starts are then exactly A's starts before p
followed by W's starts from p, and that p starts a pre-token of A.  Since
every pre-token is encoded on its own (Appendix A.1), the spliced tokens then
equal a fresh encode of X.

These tests check the claim with the oracle's own regex split, which knows
nothing of the rule: on random texts built to hit the rules' long reaches
(digit groups, whitespace and newline runs, contractions near the window
edge), and on structured cases.  They also show that the conditions are
needed: a 3-char left margin breaks GPT-2-style rules (a contraction whose
apostrophe follows a space), and without the class change cl100k-style digit
groups break.
"""
import random

import pytest
import regex

from oracle.pretok import CL100K, GPT2, split

_L, _N, _W = regex.compile(r"\p{L}"), regex.compile(r"\p{N}"), regex.compile(r"\s")
LEFT, RIGHT = 4, 5


def klass(c):
    return "L" if _L.match(c) else "N" if _N.match(c) else "W" if _W.match(c) else "O"


def starts(text, pat):
    out, pos = [], 0
    for piece in split(text, pat):
        out.append(pos)
        pos += len(piece)
    return out


def qualifies(x, a_len, w0, p, pat, left=LEFT, right=RIGHT, need_class_change=True):
    if p < w0 + left or p > a_len - right:
        return False
    return pat == GPT2 or not need_class_change or klass(x[p]) != klass(x[p - 1])


def splice_holds(a, d, w0, p, pat):
    x = a + d
    sa, sx = starts(a, pat), starts(x, pat)
    sw = [w0 + s for s in starts(x[w0:], pat)]
    return p in sa and [s for s in sa if s < p] + [s for s in sw if s >= p] == sx


ALPHA = list("asSrtTdleEvmL1279.;'\"-_ ") + [" ", " ", "\n", "\r", "\t", "　", "中", "é", "²"]


def _rand_text(rng, n):
    out = []
    while len(out) < n:
        c = rng.choice(ALPHA)
        out.extend([c] * (rng.choice([1, 2, 3, 5, 8, 13]) if rng.random() < 0.3 else 1))
    return "".join(out[:n])


@pytest.mark.parametrize("pat", [GPT2, CL100K])
def test_splice_rule_on_random_texts(pat):
    rng = random.Random(1000 + pat)
    checked = 0
    for _ in range(1500):
        a = _rand_text(rng, rng.randint(LEFT + RIGHT + 1, 28))
        d = _rand_text(rng, rng.randint(1, 8))
        x = a + d
        for w0 in range(1, len(a)):
            for p in starts(x[w0:], pat):
                p += w0
                if qualifies(x, len(a), w0, p, pat):
                    checked += 1
                    assert splice_holds(a, d, w0, p, pat), (a, d, w0, p)
    assert checked > 25_000


@pytest.mark.parametrize("pat", [GPT2, CL100K])
def test_splice_rule_on_long_runs(pat):
    # runs much longer than the margins on both sides of the window edge
    pieces = ["1234567890" * 3, " " * 17, "\n\n\n", "  \n \n  ", "abcdef'sXY'LL", "..;;--", "x" * 25,
              "　　", "中文", "\r\n\r\n", "'t'd've'RE"]
    rng = random.Random(7 + pat)
    checked = 0
    for _ in range(250):
        a = "".join(rng.choice(pieces) for _ in range(rng.randint(2, 5)))
        d = "".join(rng.choice(pieces) for _ in range(rng.randint(1, 2)))[: rng.randint(1, 12)]
        x = a + d
        for w0 in range(1, len(a), max(1, len(a) // 12)):
            for p in starts(x[w0:], pat):
                p += w0
                if qualifies(x, len(a), w0, p, pat):
                    checked += 1
                    assert splice_holds(a, d, w0, p, pat), (a, d, w0, p)
    assert checked > 1000


def test_left_margin_of_three_is_not_enough_for_gpt2():
    # the window starts at the apostrophe: on its own it reads as the
    # contraction 'll, but in the whole text the apostrophe follows a space
    a, d, w0, p = " 'llllllll \"", ".e", 1, 4
    x = a + d
    assert p in [w0 + s for s in starts(x[w0:], GPT2)]
    assert qualifies(x, len(a), w0, p, GPT2, left=3)
    assert not qualifies(x, len(a), w0, p, GPT2)
    assert not splice_holds(a, d, w0, p, GPT2)


def test_cl100k_needs_a_class_change():
    # inside a digit run the 3-digit groups count from the run start
    a, d = "x 1111111111111111 y", "z"
    x = a + d
    w0 = 4
    bad = [w0 + s for s in starts(x[w0:], CL100K)
           if qualifies(x, len(a), w0, w0 + s, CL100K, need_class_change=False)
           and not qualifies(x, len(a), w0, w0 + s, CL100K)]
    assert bad and not all(splice_holds(a, d, w0, p, CL100K) for p in bad)
