"""Text generators for the benchmark workloads.

All draws are seeded (numpy PCG64 via ``default_rng``), so a (kind, size, seed)
triple always yields the same bytes.  Shapes follow the workload list of the
project: code-like ASCII text, a code/log mix of identifier lines, numbers,
whitespace runs and punctuation, the same mix with 5 % multibyte chars, a
log-normal batch of fresh texts, and four adversarial texts.
"""
import math

import random

import numpy as np

ASCII_PUNCT = "!\"#$%&'()*+,-./:;<=>?@[\\]^_`{|}~"
assert len(ASCII_PUNCT) == 32

KEYWORDS = [
    "def", "return", "if", "else", "elif", "for", "while", "class", "import",
    "from", "int", "float", "const", "let", "var", "function", "struct", "self",
    "this", "None", "True", "False", "null", "void", "static", "public",
    "private", "fn", "pub", "mut", "match", "case", "break", "continue", "try",
    "except", "catch", "finally", "with", "async", "await", "yield", "lambda",
]
CONTRACTIONS = ["s", "t", "re", "ve", "m", "ll", "d"]

_ONSETS = list("bcdfghjklmnprstvwz") + ["ch", "sh", "th", "st", "tr", "pr", "gr", "bl", "cl"]
_VOWELS = list("aeiou") + ["ai", "ea", "ou", "io"]
_CODAS = list("nrstlmkdgp") + ["nt", "st", "ng", "ck"]


def lexicon(seed=7, size=200_000):
    """``size`` distinct lower-case words of 1-4 CV/CVC syllables, in draw
    order (the Zipf rank of a word is its index)."""
    rng = np.random.default_rng(seed)
    words, seen = [], set()
    while len(words) < size:
        k = 4096
        nsyl = rng.choice([1, 2, 3, 4], size=k, p=[0.2, 0.4, 0.3, 0.1])
        on = rng.integers(0, len(_ONSETS), size=(k, 4))
        vo = rng.integers(0, len(_VOWELS), size=(k, 4))
        has_coda = rng.random((k, 4)) < 0.35
        co = rng.integers(0, len(_CODAS), size=(k, 4))
        for i in range(k):
            w = "".join(
                _ONSETS[on[i, j]] + _VOWELS[vo[i, j]] + (_CODAS[co[i, j]] if has_coda[i, j] else "")
                for j in range(nsyl[i])
            )
            if w not in seen:
                seen.add(w)
                words.append(w)
                if len(words) == size:
                    break
    return words


_LEX_CACHE = {}


def _lex():
    if "lex" not in _LEX_CACHE:
        words = lexicon()
        ranks = np.arange(1, len(words) + 1, dtype=np.float64)
        cdf = np.cumsum(ranks ** -1.1)
        _LEX_CACHE["lex"] = (words, cdf / cdf[-1])
    return _LEX_CACHE["lex"]


class _Draw:
    """Buffered bulk random draws (numpy) for the per-token Python loop."""

    def __init__(self, seed):
        self.rng = np.random.default_rng(seed)
        self._u = np.empty(0)
        self._ui = 0

    def u(self):
        if self._ui >= len(self._u):
            self._u = self.rng.random(1 << 16)
            self._ui = 0
        v = self._u[self._ui]
        self._ui += 1
        return v

    def int(self, lo, hi):
        """Uniform integer in [lo, hi]."""
        return lo + int(self.u() * (hi - lo + 1))

    def pick(self, seq):
        return seq[int(self.u() * len(seq))]


def _word(d, words, cdf):
    return words[min(int(np.searchsorted(cdf, d.u())), len(words) - 1)]


def _identifier(d, words, cdf, accent_rate=0.0):
    """A lexicon identifier in one of several styles; optional contraction."""
    r = d.u()
    if r < 0.18:
        w = d.pick(KEYWORDS)
    else:
        style = d.u()
        if style < 0.60:
            w = _word(d, words, cdf)
        elif style < 0.80:
            w = "_".join(_word(d, words, cdf) for _ in range(d.int(2, 3)))
        elif style < 0.95:
            parts = [_word(d, words, cdf) for _ in range(d.int(2, 3))]
            w = parts[0] + "".join(p[:1].upper() + p[1:] for p in parts[1:])
        else:
            w = _word(d, words, cdf).upper()
    if accent_rate > 0.0:
        w = "".join(_accent(d) if (c.isalpha() and d.u() < accent_rate) else c for c in w)
    if d.u() < 0.01:
        suf = d.pick(CONTRACTIONS)
        if d.u() < 0.10:
            suf = suf.upper()
        w = w + "'" + suf
    return w


# Accented Latin letters U+00C0..U+024F, minus the two math signs and the long s.
_ACCENTED = [chr(c) for c in range(0xC0, 0x250) if c not in (0xD7, 0xF7, 0x17F)]


def _accent(d):
    return d.pick(_ACCENTED)


def code_text(n_bytes, seed):
    """ASCII code-like text of exactly ``n_bytes`` bytes: indented lines of
    identifiers, keywords, 1-6 digit numbers and punctuation."""
    words, cdf = _lex()
    d = _Draw(seed)
    ops = ["=", "(", ")", ",", ".", ":", ";", "+=", "==", "->", "[", "]", "{", "}", "+", "-", "*", "/", "<", ">", "!="]
    out, total = [], 0
    while total < n_bytes:
        depth = d.int(0, 3)
        line = ("\t" if d.u() < 0.2 else "    ") * depth
        toks = []
        for _ in range(d.int(1, 8)):
            r = d.u()
            if r < 0.55:
                toks.append(_identifier(d, words, cdf))
            elif r < 0.70:
                toks.append("".join(str(d.int(0, 9)) for _ in range(d.int(1, 6))))
            else:
                toks.append(d.pick(ops))
        for t in toks:
            line += t
            if d.u() < 0.6:
                line += " "
        line += "\n"
        out.append(line)
        total += len(line)
    s = "".join(out)[:n_bytes]
    b = s.encode("ascii")
    assert len(b) == n_bytes
    return b


# Nominal mean segment lengths (chars) used to turn char shares into draw
# probabilities: P(type) is proportional to share / mean length.
_MIX = [("ident", 0.70, 36.0), ("num", 0.15, 6.5), ("ws", 0.10, 4.0), ("punct", 0.05, 2.0)]


def mix_text(n_chars, seed, multibyte=False):
    """Code/log mix of exactly ``n_chars`` code points, returned as UTF-8.

    Char shares: 70 % identifier-and-keyword lines (1-8 words, single spaces,
    newline), 15 % numbers (1-12 uniform digits), 10 % whitespace runs
    (geometric length, mean 4; each char space 80 %, tab 10 %, newline 10 %),
    5 % punctuation (runs of 1-3 ASCII punctuation chars).  With
    ``multibyte``, about 5 % of chars are multibyte in equal thirds: CJK runs
    of 1-4 (U+4E00-U+9FA5), accented Latin letters inside identifiers, and
    standalone emoji (U+1F300-U+1F64F).
    """
    words, cdf = _lex()
    d = _Draw(seed)
    kinds = list(_MIX)
    if multibyte:
        # about 1.67 % of chars each: CJK runs (mean 2.5), emoji (1 char)
        kinds = kinds + [("cjk", 0.0167, 2.5), ("emoji", 0.0167, 1.0)]
    w = np.array([s / m for _, s, m in kinds])
    cum = np.cumsum(w / w.sum())
    accent_rate = 0.027 if multibyte else 0.0
    out, total = [], 0
    while total < n_chars:
        u = d.u()
        k = kinds[min(int(np.searchsorted(cum, u)), len(kinds) - 1)][0]
        if k == "ident":
            seg = " ".join(_identifier(d, words, cdf, accent_rate) for _ in range(d.int(1, 8))) + "\n"
        elif k == "num":
            seg = "".join(str(d.int(0, 9)) for _ in range(d.int(1, 12)))
        elif k == "ws":
            n = 1
            while d.u() >= 0.25:
                n += 1
            seg = "".join(" " if (r := d.u()) < 0.8 else ("\t" if r < 0.9 else "\n") for _ in range(n))
        elif k == "punct":
            seg = "".join(d.pick(ASCII_PUNCT) for _ in range(d.int(1, 3)))
        elif k == "cjk":
            seg = "".join(chr(d.int(0x4E00, 0x9FA5)) for _ in range(d.int(1, 4)))
        else:
            seg = chr(d.int(0x1F300, 0x1F64F))
        out.append(seg)
        total += len(seg)
    s = "".join(out)[:n_chars]
    assert len(s) == n_chars
    return s.encode("utf-8")


def batch_texts(n_seqs=64, median=120_000, sigma=0.29, lo=2048, hi=1_000_000, seed=40_000):
    """Log-normal batch of fresh texts from the multibyte mix.

    Length (chars) of text i: clip(round(exp(ln median + sigma * Z_i)), lo, hi)
    with Z_i standard normal (seeded); text i uses seed ``seed + i``.
    Returns (concatenated bytes, int64 offsets[n_seqs + 1]).
    """
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(n_seqs)
    lens = np.clip(np.round(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)
    parts = [mix_text(int(lens[i]), seed + 1 + i, multibyte=True) for i in range(n_seqs)]
    offsets = np.zeros(n_seqs + 1, dtype=np.int64)
    offsets[1:] = np.cumsum([len(p) for p in parts])
    return b"".join(parts), offsets


def adversarial_text(kind, n_chars=1_000_000):
    """The four adversarial texts (all ASCII, exactly ``n_chars`` bytes).

    a: one letter repeated (a single giant piece)
    b: runs of 100,000 uniform digits, each followed by a newline (seed 105)
    c: runs of 50,000 spaces, each followed by one char cycling x, 7, .
    d: letters a-z/A-Z at even positions, ASCII punctuation at odd (seed 106)
    """
    if kind == "a":
        return b"a" * n_chars
    if kind == "b":
        rng = np.random.default_rng(105)
        parts, total = [], 0
        while total < n_chars:
            digs = rng.integers(0, 10, size=100_000).astype(np.uint8) + ord("0")
            parts.append(digs.tobytes() + b"\n")
            total += 100_001
        return b"".join(parts)[:n_chars]
    if kind == "c":
        parts, total, i = [], 0, 0
        while total < n_chars:
            parts.append(b" " * 50_000 + b"x7."[i % 3:i % 3 + 1])
            total += 50_001
            i += 1
        return b"".join(parts)[:n_chars]
    if kind == "d":
        rng = np.random.default_rng(106)
        letters = np.frombuffer(b"abcdefghijklmnopqrstuvwxyzABCDEFGHIJKLMNOPQRSTUVWXYZ", dtype=np.uint8)
        punct = np.frombuffer(ASCII_PUNCT.encode(), dtype=np.uint8)
        out = np.empty(n_chars, dtype=np.uint8)
        out[0::2] = letters[rng.integers(0, 52, size=(n_chars + 1) // 2)]
        out[1::2] = punct[rng.integers(0, 32, size=n_chars // 2)]
        return out.tobytes()
    raise ValueError(kind)


# Workload table: name -> (pattern id, vocab name, description).
WORKLOADS = {
    "c1": (0, "c1", "64 KiB ASCII code-like text, GPT-2-style rules, 4,096 merges"),
    "c2": (0, "c2", "1,000,000-char code/log mix, GPT-2-style rules, 50,000 merges"),
    "c3": (1, "c3", "1,000,000-char mix with 5% multibyte, cl100k-style rules, 100,000 merges"),
    "c4": (1, "c3", "batch of 64 log-normal texts (~8M chars), cl100k-style rules, 100,000 merges"),
    "c5a": (1, "c3", "1,000,000 x 'a' (one giant piece), cl100k-style rules"),
    "c5b": (1, "c3", "100,000-digit runs, cl100k-style rules"),
    "c5c": (1, "c3", "50,000-space runs with a trailing non-space, cl100k-style rules"),
    "c5d": (1, "c3", "alternating letter/punctuation, cl100k-style rules"),
    "w100k": (0, "c2", "one 100,000-letter random word (12 letters), GPT-2-style rules, 50,000 merges"),
    "o2": (2, "c3", "1,000,000-char mix with 5% multibyte, o200k-style rules, 100,000 merges"),
    "ds": (3, "c3", "1,000,000-char mix with 5% multibyte, DeepSeek-style rules, 100,000 merges"),
}


def workload(name):
    """(bytes, offsets or None, pattern id, vocab name) of a named workload."""
    pat, voc, _ = WORKLOADS[name]
    if name == "c1":
        return code_text(65_536, 101), None, pat, voc
    if name == "c2":
        return mix_text(1_000_000, 102), None, pat, voc
    if name == "c3":
        return mix_text(1_000_000, 103, multibyte=True), None, pat, voc
    if name == "c4":
        data, off = batch_texts()
        return data, off, pat, voc
    if name.startswith("c5"):
        return adversarial_text(name[2]), None, pat, voc
    if name == "w100k":
        return random_word(100_000, 5), None, pat, voc
    if name in ("o2", "ds"):
        return mix_text(1_000_000, 103, multibyte=True), None, pat, voc
    raise ValueError(name)


def random_word(n_letters, seed, alphabet="etaoinshrdlu"):
    """One pre-token of ``n_letters`` letters drawn uniformly (Python's seeded
    ``random``): a long piece with thousands of distinct merges."""
    rng = random.Random(seed)
    return "".join(rng.choice(alphabet) for _ in range(n_letters)).encode()


# Training corpora for the three vocabularies: (generator, size, seed, rules, M).
CORPORA = {
    "c1": ("code", 1_000_000, 201, 0, 4_096),
    "c2": ("mix", 20_000_000, 202, 0, 50_000),
    "c3": ("mixmb", 50_000_000, 203, 1, 100_000),
}


def corpus(name):
    kind, size, seed, _, _ = CORPORA[name]
    if kind == "code":
        return code_text(size, seed)
    return mix_text(size, seed, multibyte=(kind == "mixmb"))
