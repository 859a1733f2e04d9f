"""Run-decomposition pre-tokenizer, written for the tests only.

An independent formulation of the two rule sets, used to pin the oracle's
sequential regex split by brute force: TokTier summary page, §4.1, says the
serial regex split can be reproduced from maximal runs of same-class chars,
the offset inside a run, a few chars of context either side and run-level
facts.  ``piece_starts`` evaluates that per-position predicate directly from
the rule tables (no regex engine); tests check it equals the regex split on
every short string over a class-covering alphabet.

Classes: L letters, N digits, WN = CR/LF, WS = other whitespace, O the rest.
The o200k-style set (pattern 2) splits letters further by case: U (Lu, Lt),
LW (Ll), B (Lm, Lo and combining marks, which go with either case).
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


_LU = regex.compile(r"[\p{Lu}\p{Lt}]")
_LL = regex.compile(r"\p{Ll}")
_LB = regex.compile(r"[\p{Lm}\p{Lo}\p{M}]")
U, LW, B = "U", "LW", "B"


def char_class2(ch):
    """o200k-style classes: U, LW, B (letter-type), N, WS, WN, O."""
    c = char_class(ch)
    if c in (WN, WS, N):
        return c
    if _LU.match(ch):
        return U
    if _LL.match(ch):
        return LW
    if _LB.match(ch):
        return B
    return O


def _is_w(c):
    return c in (WS, WN)


def piece_starts(text, pattern_id):
    """Char indices where a pre-token starts (pattern 0 GPT-2-style, 1
    cl100k-style, 2 o200k-style, 3 DeepSeek-style)."""
    if pattern_id == 2:
        return _o200k_starts(text)
    if pattern_id == 3:
        return _deepseek_starts(text)
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


def _o200k_starts(text):
    """o200k-style starts.  Letter-type chars (U, LW, B) form letter blocks;
    inside one, a new word starts at an upper-case char U when the last cased
    char of the current word is lower-case (rule A), or when it follows a B
    char, no lower-case char precedes it in the word and only upper-case
    chars follow it to the block's end (rule B: the lower-type run must take
    at least one char, so it takes the last B and leaves the upper-case tail).
    A contraction after a word belongs to it; the char after the contraction
    starts a word.  An "other" char followed by CR/LF starts a tail of CR, LF
    and '/' chars that belongs to its piece."""
    n = len(text)
    cls = [char_class2(ch) for ch in text]
    li = [c in (U, LW, B) for c in cls]
    # tails: CR/LF right after an "other" char, then CR, LF and '/' chars
    tail = [False] * n
    for i in range(1, n):
        if cls[i] == WN and cls[i - 1] == O:
            tail[i] = True
        elif tail[i - 1] and (cls[i] == WN or text[i] == "/"):
            tail[i] = True
    # contractions attached to the word before them; after[i]: a word
    # restarts.  The apostrophe right after an attached contraction cannot
    # attach (no word ends there): along back-to-back contractions attachment
    # alternates.
    def shape(a):
        one = text[a + 1] if a + 1 < n else ""
        two = text[a + 1:a + 3]
        if one.isascii() and one.lower() in ("s", "t", "m", "d"):
            return 1
        if len(two) == 2 and two.isascii() and two.lower() in ("re", "ve", "ll"):
            return 2
        return 0

    contr = [0] * n
    after = [False] * n
    in_contr = [False] * n
    for a in range(1, n - 1):
        if text[a] == "'" and li[a - 1]:
            m = shape(a)
            prev_attached = any(a - k - 1 >= 0 and contr[a - k - 1] == k for k in (1, 2))
            if m and not prev_attached:
                contr[a] = m
                for k in range(1, m + 1):
                    in_contr[a + k] = True
                if a + m + 1 < n:
                    after[a + m + 1] = True
    run_start = [0] * n
    for i in range(1, n):
        run_start[i] = run_start[i - 1] if cls[i] == cls[i - 1] else i
    wrun_end = [n] * n
    for i in range(n - 2, -1, -1):
        wrun_end[i] = wrun_end[i + 1] if (_is_w(cls[i]) and _is_w(cls[i + 1]) and
                                          (cls[i] == WS) == (cls[i + 1] == WS)) else i + 1

    def prev_cased_lower(i):
        # the last cased char of the current word before i is lower-case
        k = i - 1
        while k >= 0 and cls[k] == B and not after[k]:
            k -= 1
        return k >= 0 and cls[k] == LW

    def only_upper_to_end(i):
        k = i
        while k < n and cls[k] == U:
            k += 1
        return k == n or not li[k]

    starts = [0] if n else []
    for i in range(1, n):
        c, p = cls[i], cls[i - 1]
        if c == N:
            b = p != N or (i - run_start[i]) % 3 == 0
        elif c == WN:
            b = not (_is_w(p) or p == O)
        elif c == WS:
            if not _is_w(p):
                b = True
            elif p == WN:
                s = run_start[i - 1]
                ends_run = wrun_end[i] == n or not _is_w(cls[wrun_end[i]])
                b = ends_run or (s > 0 and cls[s - 1] == O)
            else:
                b = i + 1 < n and not _is_w(cls[i + 1])
        elif c == O:
            if tail[i]:
                b = False
            elif text[i - 1] == " ":
                b = False
            elif p == O:
                b = tail[i - 1]
            elif li[i - 1] and contr[i]:
                b = False
            else:
                b = True
        else:  # letter-type
            if in_contr[i]:
                b = False
            elif li[i - 1]:
                b = after[i] or (c == U and prev_cased_lower(i)) or \
                    (c == U and p == B and not prev_cased_lower(i) and only_upper_to_end(i))
            elif p == WS:
                b = False
            elif p == O:
                if tail[i - 1]:
                    b = True
                else:
                    b = i >= 2 and ((cls[i - 2] == O and not tail[i - 2]) or text[i - 2] == " ")
            else:
                b = True
        if b:
            starts.append(i)
    return starts


_LM = regex.compile(r"[\p{L}\p{M}]")
_PS = regex.compile(r"[\p{P}\p{S}]")
LM, PS = "LM", "PS"


def char_class3(ch):
    """DeepSeek-style classes: LM (letters and marks), PS (punctuation and
    symbols), N, WS, WN, O (the rest)."""
    c = char_class(ch)
    if c in (WN, WS, N):
        return c
    if _LM.match(ch):
        return LM
    if _PS.match(ch):
        return PS
    return O


def _deepseek_starts(text):
    """DeepSeek-style starts.  Digit groups and CJK/kana runs cut the text
    into segments first (each starts a piece, and a segment's end is the end
    of text for the rules inside it).  Inside a segment: an ASCII
    punctuation/symbol char that starts a piece and is followed by ASCII
    letters takes those letters (D1); otherwise letters and marks form words
    with one optional leading char (whitespace, "other"); punctuation and
    symbols form runs (with one leading space) that take the CR/LF chars after
    them; whitespace follows the same rules as cl100k-style; "other" chars
    no rule takes are pieces of their own, joined while they follow each other."""
    n = len(text)
    cls = [char_class3(ch) for ch in text]
    cjk = [0x4E00 <= ord(ch) <= 0x9FA5 or 0x3040 <= ord(ch) <= 0x30FF for ch in text]
    al = [ch.isascii() and ch.isalpha() for ch in text]
    ap1 = [ch.isascii() and bool(_PS.match(ch)) for ch in text]
    seg = [False] * n
    dig = 0
    for i in range(n):
        if cls[i] == N:
            dig = dig + 1 if i > 0 and cls[i - 1] == N else 0
            seg[i] = dig % 3 == 0
        else:
            seg[i] = i == 0 or cls[i - 1] == N or cjk[i] != cjk[i - 1]
    if n:
        seg[0] = True
    same = [i > 0 and not seg[i] for i in range(n)]  # i - 1 lies in i's segment

    def nxt(i):  # class of the next char of the segment, or None
        return cls[i + 1] if i + 1 < n and same[i + 1] else None

    d1s = [ap1[i] and i + 1 < n and same[i + 1] and al[i + 1] and
           (not same[i] or (cls[i - 1] != PS and text[i - 1] != " ")) for i in range(n)]
    d1l = [False] * n
    for i in range(n):
        d1l[i] = al[i] and same[i] and (d1s[i - 1] or d1l[i - 1])
    wrun_end = [n] * n  # end of the whitespace run of the same kind (WS or WN) in the segment
    for i in range(n - 1, -1, -1):
        if i + 1 < n and same[i + 1] and cls[i + 1] == cls[i]:
            wrun_end[i] = wrun_end[i + 1]
        else:
            wrun_end[i] = i + 1
    run_start = [0] * n
    for i in range(n):
        run_start[i] = run_start[i - 1] if same[i] and cls[i] == cls[i - 1] else i

    starts = []
    for i in range(n):
        if seg[i]:
            starts.append(i)
            continue
        c, p = cls[i], cls[i - 1]
        if c == N:
            b = False
        elif c == LM:
            if p == LM:
                b = d1l[i - 1] and not al[i]
            elif p == PS:
                b = not (d1s[i - 1] and al[i])
            else:
                b = p == WN
        elif c == PS:
            b = p != PS and text[i - 1] != " "
        elif c == WN:
            b = not (_is_w(p) or p == PS)
        elif c == WS:
            if not _is_w(p):
                b = True
            elif p == WN:
                e = wrun_end[i]
                ends_run = e == n or not same[e] or not _is_w(cls[e])
                s0 = run_start[i - 1]
                b = ends_run or (same[s0] and cls[s0 - 1] == PS)
            else:
                q = nxt(i)
                b = q is not None and not _is_w(q)
        else:  # O
            b = p != O or nxt(i) == LM
        if b:
            starts.append(i)
    return starts
