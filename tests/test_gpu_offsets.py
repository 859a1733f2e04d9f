"""Device-side byte-offset export (tt_encode_offsets) against the oracle.

TokTier summary page, Path C of §8 and Appendix E: the GPU returns each
token's byte span along with its id.  Every case compares the ids and the T+1
byte offsets with oracle.bpe.encode_offsets element by element, and the ids
with tt_encode's.  The cases cover every copy path of the emission kernel
(pieces of <= 8 tokens, of <= 64, and longer pieces cut into 4,096-token
chunks, with chunk counts around the chunk edges), batches with empty texts,
multi-byte text, no merges, and the data errors.
"""
import os
import random

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from oracle.bpe import Vocab, encode_offsets as oracle_offsets  # noqa: E402
from oracle.pretok import CL100K, GPT2  # noqa: E402
from synth import code_text, mix_text  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHUNK = 4096  # tokens per work item of a long piece in the emission kernel


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def dev(data):
    return torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda() if len(data) else torch.empty(
        0, dtype=torch.uint8, device="cuda")


def load(name_or_merges, pattern):
    merges = (np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % name_or_merges))
              if isinstance(name_or_merges, str) else name_or_merges)
    tt.load(merges, pattern_id=pattern)
    return Vocab(merges)


def check(data, v, pattern, offsets=None):
    x = dev(data)
    if offsets is None:
        ids, starts = tt.encode_offsets(x)
        plain = tt.encode(x)
    else:
        off = torch.tensor(offsets, dtype=torch.int64, device="cuda")
        ids, starts, cnt = tt.encode_offsets(x, off)
        plain, plain_cnt = tt.encode_batch(x, off)
        assert cnt.tolist() == plain_cnt.tolist()
    ids, starts = ids.cpu().numpy(), starts.cpu().numpy()
    wi, ws, wc = oracle_offsets(data, offsets, v, pattern)
    assert np.array_equal(ids, np.asarray(wi, dtype=np.int32))
    assert np.array_equal(plain.cpu().numpy(), ids)
    ws = np.asarray(ws, dtype=np.int32)
    if not np.array_equal(starts, ws):
        d = np.nonzero(starts[:len(ws)] != ws[:len(starts)])[0]
        raise AssertionError("%d vs %d offsets; first difference at %s" % (len(starts), len(ws), d[:5]))
    if offsets is not None:
        assert cnt.tolist() == wc


@pytest.mark.parametrize("pattern", [GPT2, CL100K])
def test_offsets_code_and_multibyte_text(pattern):
    v = load("c1", pattern)
    say("offsets code_text 64KiB seed 21 + mix 40K multibyte seed 22, pattern", pattern)
    check(code_text(65_536, 21), v, pattern)
    check(mix_text(40_000, 22, multibyte=True), v, pattern)


def test_offsets_empty_and_one_byte():
    v = load("c1", GPT2)
    say("offsets empty / one byte")
    check(b"", v, GPT2)
    check(b"q", v, GPT2)
    check(b"\xe4\xb8\xad", v, GPT2)


def test_offsets_batch_with_empty_texts():
    v = load("c3", CL100K)
    texts = [b"", code_text(5_000, 23), b"", mix_text(3_000, 24, multibyte=True), b" ", b"a" * 20_000, b""]
    offs = [0]
    for t in texts:
        offs.append(offs[-1] + len(t))
    say("offsets batch of", len(texts), "texts,", offs[-1], "bytes")
    check(b"".join(texts), v, CL100K, offs)


@pytest.mark.parametrize("run", [8, 9, 64, 65, CHUNK - 1, CHUNK, CHUNK + 1, 2 * CHUNK, 2 * CHUNK + 5, 3 * CHUNK + 100,
                                 16 * CHUNK + 7])
def test_offsets_copy_paths_and_chunk_edges(run):
    # with the c3 vocabulary "aa" is no merge, so a run of r letters a is one
    # pre-token of r one-byte tokens: r picks the copy path
    v = load("c3", CL100K)
    say("offsets a-run of", run)
    check(b"x = " + b"a" * run + b" + 1\n", v, CL100K)


def test_offsets_several_long_pieces_of_mixed_token_lengths():
    merges = [(97, 98), (99, 100), (256, 257), (97, 97), (259, 259), (258, 97), (260, 98)]
    v = load(np.asarray(merges, dtype=np.int32), GPT2)
    rng = random.Random(25)
    parts = []
    for k in range(5):
        parts.append(bytes(rng.choice(b"abcd") for _ in range(rng.randint(20_000, 60_000))))
        parts.append(b" %d, " % k)
    data = b"".join(parts)
    say("offsets 5 long letter pieces,", len(data), "bytes")
    check(data, v, GPT2)


def test_offsets_no_merges():
    v = load(np.zeros((0, 2), dtype=np.int32), CL100K)
    data = mix_text(20_000, 26, multibyte=True)
    say("offsets no merges,", len(data), "bytes")
    ids, starts = tt.encode_offsets(dev(data))
    assert starts.cpu().numpy().tolist() == list(range(len(data) + 1))
    check(data, v, CL100K)


def test_offsets_data_errors():
    load("c1", GPT2)
    say("offsets invalid UTF-8 / bad batch offsets")
    with pytest.raises(tt.TTError) as e:
        tt.encode_offsets(dev(b"abc \xff def"))
    assert e.value.code == tt.TT_EUTF8
    x = dev(b"hello world")
    with pytest.raises(tt.TTError) as e:
        tt.encode_offsets(x, torch.tensor([0, 7, 3, 11], dtype=torch.int64, device="cuda"))
    assert e.value.code == tt.TT_EOFFSETS
