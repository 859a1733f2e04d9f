"""Oracle pre-tokenizer: sequential regex split (the G stage of F = E* o G).

TokTier summary page, §3.2 and Appendix A.1: GPT-style tokenization first cuts
the text into pre-tokens with an ordered regex (leftmost alternative that
matches wins, greedy quantifiers with backtracking), then encodes each piece on
its own.  The pages name the rule families but never print the patterns, so
the four rule sets below are this project's renderings of the families' known
features:

  pattern 0, GPT-2-style: contractions (lower case), letters, digits,
  punctuation, whitespace with the "not followed by a non-space" lookahead.

  pattern 1, cl100k-style: contractions with ASCII-only case folding, letters
  with one optional leading non-letter/non-digit/non-newline char, digit groups
  of one to three, punctuation that swallows the CR/LF chars after it,
  whitespace up to the last CR/LF, then the lookahead rule.

  pattern 2, o200k-style: words split by letter case, contractions attached
  to the word, digit groups, "other" runs with CR/LF/'/' tails, whitespace
  rules as cl100k-style.

  pattern 3, DeepSeek-style: digit groups and CJK/kana runs cut out first, then
  punctuation/letter/whitespace rules on every piece by itself.

Character sets (pinned by tests against the ``regex`` module's own classes):
  L  = \\p{L}    N = \\p{N}    (Unicode tables of the ``regex`` module)
  W  = the 25 code points with the Unicode White_Space property.  U+001C..U+001F
       are *not* whitespace here (``str.isspace`` disagrees; we do not use it).
  O  = everything else.

Invalid UTF-8 is an error (raised by the strict decoder), never replaced.
"""
import regex

# The Unicode White_Space property, spelled out (25 code points).
WHITESPACE_CPS = (
    [0x09, 0x0A, 0x0B, 0x0C, 0x0D, 0x20, 0x85, 0xA0, 0x1680]
    + list(range(0x2000, 0x200B))
    + [0x2028, 0x2029, 0x202F, 0x205F, 0x3000]
)
_W = "\\t\\n\\x0b\\x0c\\r \\x85\\xa0\\u1680\\u2000-\\u200a\\u2028\\u2029\\u202f\\u205f\\u3000"
W_CLASS = "[" + _W + "]"          # one whitespace char
NOT_W_CLASS = "[^" + _W + "]"     # one non-whitespace char
O_CLASS = "[^" + _W + "\\p{L}\\p{N}]"  # neither whitespace, letter nor digit

GPT2 = 0
CL100K = 1
O200K = 2
DEEPSEEK = 3

# GPT-2-style, alternatives in priority order:
#   G1 apostrophe contraction (lower case only)
#   G2 optional space + letters      G3 optional space + digits
#   G4 optional space + "other" run
#   G5 whitespace not followed by a non-whitespace char   G6 whitespace
_GPT2_RULES = [
    "'(?:s|t|re|ve|m|ll|d)",
    " ?\\p{L}+",
    " ?\\p{N}+",
    " ?" + O_CLASS + "+",
    W_CLASS + "+(?!" + NOT_W_CLASS + ")",
    W_CLASS + "+",
]

# cl100k-style, alternatives in priority order:
#   C1 contraction, ASCII case-insensitive (explicit [sS] etc, no Unicode folding)
#   C2 one optional char that is not CR/LF/letter/digit, then letters
#   C3 one to three digits
#   C4 optional space, "other" run, then any CR/LF chars
#   C5 whitespace up to and including the last CR/LF of the whitespace run
#   C6 whitespace not followed by a non-whitespace char   C7 whitespace
_CL100K_RULES = [
    "'(?:[sS]|[tT]|[rR][eE]|[vV][eE]|[mM]|[lL][lL]|[dD])",
    "[^\\r\\n\\p{L}\\p{N}]?\\p{L}+",
    "\\p{N}{1,3}",
    " ?" + O_CLASS + "+[\\r\\n]*",
    W_CLASS + "*[\\r\\n]+",
    W_CLASS + "+(?!" + NOT_W_CLASS + ")",
    W_CLASS + "+",
]

# o200k-style, alternatives in priority order.  Letters are split by case:
# "upper-type" chars are Lu, Lt, Lm, Lo and combining marks, "lower-type"
# chars Ll, Lm, Lo and marks (so modifier/other letters and marks go with
# either case).  Reading: marks count as letter-type chars only, never as
# "other" chars, so neither the optional leading char nor the "other" run
# takes one.
#   Q1 one optional char that is not CR/LF/letter/mark/digit, upper-type
#      chars, then one or more lower-type chars, then an optional contraction
#      (ASCII case-insensitive, attached to the word)
#   Q2 the same with one or more upper-type chars, then lower-type chars
#   Q3 one to three digits
#   Q4 optional space, "other" run, then any CR, LF and '/' chars
#   Q5 whitespace up to and including the last CR/LF run of the whitespace run
#   Q6 whitespace not followed by a non-whitespace char   Q7 whitespace
_UPPER_T = "[\\p{Lu}\\p{Lt}\\p{Lm}\\p{Lo}\\p{M}]"
_LOWER_T = "[\\p{Ll}\\p{Lm}\\p{Lo}\\p{M}]"
_LEAD = "[^\\r\\n\\p{L}\\p{M}\\p{N}]?"
_O_CLASS_M = "[^" + _W + "\\p{L}\\p{M}\\p{N}]"
_CONTRACTION = "(?:'(?:[sS]|[tT]|[rR][eE]|[vV][eE]|[mM]|[lL][lL]|[dD]))?"
_O200K_RULES = [
    _LEAD + _UPPER_T + "*" + _LOWER_T + "+" + _CONTRACTION,
    _LEAD + _UPPER_T + "+" + _LOWER_T + "*" + _CONTRACTION,
    "\\p{N}{1,3}",
    " ?" + _O_CLASS_M + "+[\\r\\n/]*",
    W_CLASS + "*[\\r\\n]+",
    W_CLASS + "+(?!" + NOT_W_CLASS + ")",
    W_CLASS + "+",
]

# DeepSeek-style: three splits in a row, each cutting every piece the one
# before left and keeping both what it matched and what lay between matches
# as pieces ("isolated" splitting):
#   S1 digit groups of one to three
#   S2 runs of CJK unified ideographs (U+4E00..U+9FA5), hiragana and katakana
#      (U+3040..U+30FF)
#   S3 the rule set below, on each piece by itself (a piece's end is the
#      end of text for the lookahead); chars no rule takes stay pieces
#   D1 an ASCII punctuation or symbol char, then ASCII letters
#   D2 one optional char that is not CR/LF/letter/punctuation/symbol, then
#      letters and marks
#   D3 optional space, a punctuation/symbol run, then any CR/LF chars
#   D4 whitespace up to and including the last CR/LF run
#   D5 whitespace not followed by a non-whitespace char   D6 whitespace
_ASCII_PS = "[!-/:-@\\[-`{-~]"
_DEEPSEEK_STAGES = [
    "\\p{N}{1,3}",
    "[\\u4e00-\\u9fa5\\u3040-\\u30ff]+",
    "|".join([
        _ASCII_PS + "[A-Za-z]+",
        "[^\\r\\n\\p{L}\\p{P}\\p{S}]?[\\p{L}\\p{M}]+",
        " ?[\\p{P}\\p{S}]+[\\r\\n]*",
        W_CLASS + "*[\\r\\n]+",
        W_CLASS + "+(?!" + NOT_W_CLASS + ")",
        W_CLASS + "+",
    ]),
]

RULES = {GPT2: _GPT2_RULES, CL100K: _CL100K_RULES, O200K: _O200K_RULES}
PATTERNS = {k: "|".join(v) for k, v in RULES.items()}
_COMPILED = {k: regex.compile(v, regex.VERSION0) for k, v in PATTERNS.items()}
_STAGES = {DEEPSEEK: [regex.compile(p, regex.VERSION0) for p in _DEEPSEEK_STAGES]}


def _isolate(pieces, rx):
    """One isolating split: every match and every non-empty stretch between
    matches (or before the first / after the last) becomes a piece."""
    out = []
    for p in pieces:
        pos = 0
        for m in rx.finditer(p):
            if m.start() > pos:
                out.append(p[pos:m.start()])
            out.append(m.group())
            pos = m.end()
        if pos < len(p):
            out.append(p[pos:])
    return out


def split(text, pattern_id):
    """Split a str into pre-tokens with the ordered rule set ``pattern_id``.

    Plain left-to-right ``finditer``: each match starts where the previous one
    ended.  The rule sets match every char, so the pieces tile the text.
    """
    if pattern_id in _STAGES:
        pieces = [text] if text else []
        for rx in _STAGES[pattern_id]:
            pieces = _isolate(pieces, rx)
    else:
        pieces = [m.group() for m in _COMPILED[pattern_id].finditer(text)]
    if "".join(pieces) != text or any(p == "" for p in pieces):
        raise AssertionError("rule set did not tile the text")
    return pieces


def split_bytes(data, pattern_id):
    """Split UTF-8 bytes; returns (pieces as bytes, byte offset of each piece).

    Raises UnicodeDecodeError on invalid UTF-8 (strict decoding).
    """
    text = bytes(data).decode("utf-8", errors="strict")
    pieces = split(text, pattern_id)
    out, starts, pos = [], [], 0
    for p in pieces:
        b = p.encode("utf-8")
        out.append(b)
        starts.append(pos)
        pos += len(b)
    return out, starts


def piece_starts_batch(data, offsets, pattern_id):
    """Byte offsets (into the concatenation) of every piece of every sequence.

    Each sequence ``data[offsets[s]:offsets[s+1]]`` is an independent text: its
    end is end-of-text for the lookahead rules and no piece crosses it.
    """
    starts = []
    for s in range(len(offsets) - 1):
        a, b = offsets[s], offsets[s + 1]
        _, st = split_bytes(data[a:b], pattern_id)
        starts.extend(a + x for x in st)
    return starts
