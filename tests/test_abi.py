"""Host-side checks of libtt (no GPU needed).

  * the library loads and exports every function include/tt.h declares;
  * the compiled Unicode class table equals the regex module's classes on all
    1,114,112 code points (the one pinned Unicode version; TokTier summary page
    §5.2 reports a Unicode-version mismatch that mis-split 9,700 code points);
  * tt_load_bpe rejects bad arguments and inconsistent tables before touching
    the device; encode entry points reject bad arguments.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import regex

import exact_byte_level_amd as tt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "tt.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^(?:int|void|const char\*)\s+(tt_\w+)\(", src, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert names == sorted(["tt_load_bpe", "tt_load_bpe_ex", "tt_reserve", "tt_encode", "tt_encode_noalloc", "tt_encode_batch", "tt_pretokenize", "tt_encode_offsets",
                            "tt_session_create", "tt_session_destroy", "tt_session_reset", "tt_session_append",
                            "tt_session_view", "tt_session_read",
                            "tt_char_class", "tt_profile", "tt_profile_read", "tt_free", "tt_strerror"])
    lib = ctypes.CDLL(tt.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_unicode_table_matches_regex_all_code_points():
    tests = [(1, r"[\p{Lu}\p{Lt}]"), (2, r"\p{Ll}"), (3, r"[\p{Lm}\p{Lo}]"), (4, r"\p{M}"), (5, r"\p{N}"),
             (6, r"\s"), (7, r"\p{P}"), (8, r"\p{S}")]
    tests = [(k, regex.compile(t)) for k, t in tests]
    cls = tt.char_class
    diffs = []
    for cp in range(0x110000):
        if 0xD800 <= cp <= 0xDFFF:
            assert cls(cp) == -1
            continue
        c = chr(cp)
        want = next((k for k, t in tests if t.match(c)), 0)
        if cls(cp) != want:
            diffs.append(cp)
    assert diffs == []
    assert cls(0x110000) == -1
    # code points added in Unicode 14-17 are letters in the pinned tables
    for cp in (0x9FFD, 0x31350, 0x2EBF0, 0x1E5D0, 0x323B0, 0x16EA0):
        assert cls(cp) in (1, 2, 3)
    # a few fixed points of the classes
    assert [cls(ord(c)) for c in "Aa\u01c5\u02b0\u0301\u00b2 .$\x00"] == [1, 2, 1, 3, 4, 5, 6, 7, 8, 0]


def test_load_rejects_bad_tables_without_device():
    lib = tt.lib()

    def load(merges, ranks=None, pattern=0):
        m = np.ascontiguousarray(np.asarray(merges, dtype=np.int32).reshape(-1, 2))
        r = None if ranks is None else np.ascontiguousarray(np.asarray(ranks, dtype=np.int32))
        return lib.tt_load_bpe(m.ctypes.data, None if r is None else r.ctypes.data, len(m), pattern)

    assert load([(97, 98)], pattern=4) == tt.TT_EINVAL
    assert load([(97, 256)]) == tt.TT_ETABLE              # operand made later
    assert load([(97, 98), (97, 98)]) == tt.TT_ETABLE     # duplicate pair
    assert load([(97, 98), (98, 99)], ranks=[0, 0]) == tt.TT_ETABLE  # ranks not a permutation
    assert load([(97, 98), (98, 99)], ranks=[0, 2]) == tt.TT_ETABLE
    assert load([(97, 257), (98, 99)], ranks=[1, 0]) == tt.TT_ETABLE  # 257 = rank 1 itself
    assert lib.tt_load_bpe(None, None, -1, 0) == tt.TT_EINVAL
    m = np.ascontiguousarray(np.asarray([(97, 98)], dtype=np.int32))
    assert lib.tt_load_bpe_ex(m.ctypes.data, None, 1, 0, 2) == tt.TT_EINVAL  # unknown flag
    # with the whole-word rule, a token longer than 2048 bytes is refused:
    # a, aa, aaaa, ... up to 4096 letters
    chain = np.ascontiguousarray(np.asarray([(97, 97)] + [(256 + i, 256 + i) for i in range(11)], dtype=np.int32))
    assert lib.tt_load_bpe_ex(chain.ctypes.data, None, len(chain), 0, tt.LOAD_IGNORE_MERGES) == tt.TT_ETABLE


def test_encode_rejects_bad_arguments():
    lib = tt.lib()
    stream = ctypes.c_void_p(0)
    assert lib.tt_encode(None, -1, None, None, stream) == tt.TT_EINVAL
    assert lib.tt_encode_batch(None, 0, None, 1, None, None, stream) == tt.TT_EINVAL
    assert lib.tt_pretokenize(None, 5, None, 1, None, None, stream) == tt.TT_EINVAL
    assert tt.strerror(tt.TT_EUTF8) == "input is not valid UTF-8"
