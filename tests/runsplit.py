"""Run-decomposition pre-tokenizer, written for the tests only.

An independent formulation of the two rule sets, used to pin the oracle's
sequential regex split by brute force: TokTier summary page, §4.1, says the
serial regex split can be reproduced from maximal runs of same-class chars,
the offset inside a run, a few chars of context either side and run-level
facts.  ``piece_starts`` evaluates that per-position predicate directly from
the rule tables (no regex engine); tests check it equals the regex split on
every short string over a class-covering alphabet.

Classes: L letters, N digits, WN = CR/LF, WS = other whitespace, O the rest.
"""
import regex

_L = regex.compile(r"\p{L}")
_N = regex.compile(r"\p{N}")
WHITE = set(chr(c) for c in [0x09, 0x0A, 0x0B, 0x0C, 0x0D, 0x20, 0x85, 0xA0, 0x1680, 0x2028,
                             0x2029, 0x202F, 0x205F, 0x3000] + list(range(0x2000, 0x200B)))
L, N, O, WS, WN = "L", "N", "O", "WS", "WN"


def char_class(ch):
    if ch in "\r\n":
        return WN
    if ch in WHITE:
        return WS
    if _L.match(ch):
        return L
    if _N.match(ch):
        return N
    return O


def _is_w(c):
    return c in (WS, WN)


def piece_starts(text, pattern_id):
    """Char indices where a pre-token starts (pattern 0 GPT-2-style, 1 cl100k)."""
    n = len(text)
    cls = [char_class(ch) for ch in text]
    run_start = [0] * n
    for i in range(1, n):
        run_start[i] = run_start[i - 1] if cls[i] == cls[i - 1] else i
    run_end = [n] * n
    for i in range(n - 2, -1, -1):
        run_end[i] = run_end[i + 1] if cls[i] == cls[i + 1] else i + 1

    folds = (lambda s: s.lower()) if pattern_id == 1 else (lambda s: s)

    def apostrophe_starts_piece(q):
        # the apostrophe at q is a one-char "other" run that no space absorbs
        return text[q] == "'" and (q == 0 or (cls[q - 1] != O and text[q - 1] != " "))

    def contraction_len(a):
        """Length of the contraction suffix matched at letter position a, or 0."""
        if a < 1 or not apostrophe_starts_piece(a - 1):
            return 0
        one = text[a]
        if one.isascii() and folds(one) in ("s", "t", "m", "d"):
            return 1
        two = text[a:a + 2]
        if len(two) == 2 and two.isascii() and folds(two) in ("re", "ve", "ll"):
            return 2
        return 0

    def after_contraction(i):
        for m in (1, 2):
            a = i - m
            if a >= 1 and text[a - 1] == "'" and contraction_len(a) == m:
                return True
        return False

    starts = []
    for i in range(n):
        if i == 0:
            starts.append(0)
            continue
        c, p = cls[i], cls[i - 1]
        b = 0
        if pattern_id == 0:
            if _is_w(c):
                if not _is_w(p):
                    b = 1
                else:
                    b = 1 if (i + 1 < n and not _is_w(cls[i + 1])) else 0
            elif p == c:
                b = 1 if (c == L and after_contraction(i)) else 0
            elif text[i - 1] == " ":
                b = 0
            elif c == L and contraction_len(i) > 0:
                b = 0
            else:
                b = 1
        else:
            if c == N:
                b = 1 if (p != N or (i - run_start[i]) % 3 == 0) else 0
            elif c == L:
                if p == L:
                    b = 1 if after_contraction(i) else 0
                elif p == WS:
                    b = 0
                elif p == O:
                    b = 0 if (i - 2 < 0 or (cls[i - 2] != O and text[i - 2] != " ")) else 1
                else:
                    b = 1
            elif c == O:
                if p == O:
                    b = 0
                else:
                    b = 0 if text[i - 1] == " " else 1
            elif c == WN:
                if _is_w(p):
                    b = 0
                else:
                    b = 0 if p == O else 1
            else:  # WS
                if not _is_w(p):
                    b = 1
                elif p == WN:
                    e = run_end[i]
                    ends_run = e == n or not _is_w(cls[e])
                    s = run_start[i - 1]
                    absorbed = s > 0 and cls[s - 1] == O
                    b = 1 if (ends_run or absorbed) else 0
                else:
                    b = 1 if (i + 1 < n and not _is_w(cls[i + 1])) else 0
        if b:
            starts.append(i)
    return starts
