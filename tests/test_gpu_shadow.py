"""The shadow verifier around the GPU encodes (TokTier summary page, §3 shadow
branch and §4.3 runtime), with the oracle as the standard tokenizer.

  * every call checked (the pages' offline rate): single texts and a batch
    from the HIP path give no finding;
  * a corruption planted in the device ids after the encode is found at its
    index;
  * an asynchronous encode on a side stream whose buffers the caller reuses
    right after the call: the check sees the ids of the call, not the reuse.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from exact_byte_level_amd.shadow import ShadowVerifier  # noqa: E402
from oracle.bpe import Vocab, encode as oracle_encode  # noqa: E402
from oracle.pretok import CL100K, GPT2  # noqa: E402
from synth import code_text, mix_text  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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


def setup(name, pattern):
    merges = np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % name))
    tt.load(merges, pattern_id=pattern)
    v, memo = Vocab(merges), {}
    return v, (lambda b: oracle_encode(bytes(b), v, pattern, memo))


@pytest.mark.parametrize("pattern", [GPT2, CL100K])
def test_every_call_checked_no_findings(pattern):
    v, ref = setup("c1", pattern)
    say("shadow rate 1: 6 texts + batch of 5, pattern", pattern)
    texts = [code_text(20_000, 31), mix_text(30_000, 32), mix_text(15_000, 33, multibyte=True), b"", b"a", b" \n"]
    with ShadowVerifier(ref, rate=1.0) as sv:
        for t in texts:
            sv.encode(dev(t))
        parts = [mix_text(5_000, 40 + i, multibyte=i % 2 == 1) for i in range(4)] + [b""]
        off = torch.tensor(np.cumsum([0] + [len(p) for p in parts]), dtype=torch.int64, device="cuda")
        sv.encode_batch(dev(b"".join(parts)), off)
        sv.drain()
        st = sv.stats()
    assert st["checked"] == len(texts) + 1 and st["texts"] == len(texts) + len(parts)
    assert st["mismatches"] == 0, sv.quarantine[:1]


def test_planted_device_corruption_is_found():
    v, ref = setup("c2", GPT2)
    say("shadow: corruption planted at id 17 of a 20K-char mix")

    def corrupt(x):
        ids = tt.encode(x).clone()
        ids[17] = (ids[17] + 1) % (256 + len(v.merges))
        return ids

    t = mix_text(20_000, 51)
    with ShadowVerifier(ref, rate=1.0, encoder=corrupt) as sv:
        sv.encode(dev(t))
        sv.drain()
    (s,) = sv.quarantine
    assert s.first_diff == 17 and s.data == t and s.ref_ids == ref(t)


def test_async_call_snapshot_survives_buffer_reuse():
    v, ref = setup("c2", GPT2)
    say("shadow: encode_into on a side stream, buffers reused after the call")
    t = mix_text(200_000, 52)
    x = dev(t)
    out = torch.empty(x.numel(), dtype=torch.int32, device="cuda")
    out_n = torch.empty(1, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with ShadowVerifier(ref, rate=1.0) as sv:
        with torch.cuda.stream(side):
            tt.encode_into(x, out, out_n, stream=side)
            assert sv.observe(x, out, n_ids=out_n, stream=side)
            out.fill_(-1)                  # the caller reuses its buffers at once
            out_n.fill_(0)
            x.fill_(ord("z"))
        side.synchronize()
        sv.drain()
        st = sv.stats()
    assert st["checked"] == 1 and st["mismatches"] == 0, sv.quarantine[:1]


def test_data_error_agrees_with_a_failing_reference():
    v, ref = setup("c1", GPT2)
    say("shadow: invalid UTF-8 through encode_into (negative count)")
    bad = b"abc \xff def"
    x = dev(bad)
    out = torch.empty(x.numel(), dtype=torch.int32, device="cuda")
    out_n = torch.empty(1, dtype=torch.int64, device="cuda")
    with ShadowVerifier(ref, rate=1.0) as sv:
        tt.encode_into(x, out, out_n)
        sv.observe(x, out, n_ids=out_n)
        sv.drain()
        assert int(out_n.item()) == tt.TT_EUTF8
        assert sv.stats()["mismatches"] == 0
    # a standard tokenizer that accepts the bytes disagrees with the error
    with ShadowVerifier(lambda b: list(b), rate=1.0) as sv:
        tt.encode_into(x, out, out_n)
        sv.observe(x, out, n_ids=out_n)
        sv.drain()
        (s,) = sv.quarantine
        assert "error" in s.error and s.first_diff == 0
