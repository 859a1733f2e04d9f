"""Host logic of the shadow verifier (exact_byte_level_amd.shadow), on the CPU.

TokTier summary page, §3 (shadow branch), §4.3 (runtime: background thread,
random sampling, mismatching samples kept for offline reproduction, 100 %
offline and 5 % online) and §5.8 (injected substitutions, deletions and
shifted splits).  The encoder under test here is the oracle with faults
planted into its output, and the standard tokenizer is the oracle itself, so
every expected finding is known in advance:
  * a faithful encoder yields no finding at any rate;
  * each planted fault is found at rate 1, at the index where it was planted;
  * a batch reports only the faulty text, with indices inside that text;
  * a quarantined sample written to disk reproduces offline;
  * with every call faulty, the call of the first finding is geometric in the
    rate: P(found within k calls) = 1 - (1 - rate)^k, which at the pages'
    5 % and 42 calls is 0.885 (§5.8 reports 90 % within 42 requests);
  * a full queue drops samples instead of blocking the caller.
"""
import os
import threading

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from exact_byte_level_amd.shadow import ShadowVerifier, first_difference, load_sample  # noqa: E402
from oracle.bpe import Vocab, encode as oracle_encode  # noqa: E402
from oracle.pretok import GPT2  # noqa: E402
from synth import code_text  # noqa: E402

DATA = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "data")


@pytest.fixture(scope="module")
def vocab():
    return Vocab(np.load(os.path.join(DATA, "vocab_c1.npy")))


@pytest.fixture(scope="module")
def texts():
    full = code_text(24_000, 7)
    return [full[i * 3000:(i + 1) * 3000] for i in range(8)]


def _u8(b):
    return torch.frombuffer(bytearray(b), dtype=torch.uint8) if len(b) else torch.empty(0, dtype=torch.uint8)


def _ids(x):
    return torch.tensor(x, dtype=torch.int32)


def _reference(vocab):
    memo = {}
    return lambda b: oracle_encode(bytes(b), vocab, GPT2, memo)


# the three fault classes of §5.8, planted at token k of the true ids
def substitute(ids, k, vocab):
    out = list(ids)
    out[k] = (out[k] + 1) % (256 + len(vocab.merges))
    return out


def delete(ids, k, vocab):
    return list(ids[:k]) + list(ids[k + 1:])


def shift_split(ids, k, vocab):
    """Token k (a merged token) replaced by the pair it was merged from: the
    same bytes, cut at another place."""
    t = ids[k]
    x, y = vocab.merges[t - 256]
    return list(ids[:k]) + [x, y] + list(ids[k + 1:])


def _first_merged(ids, start):
    return next(i for i in range(start, len(ids)) if ids[i] >= 256)


def test_first_difference():
    assert first_difference([1, 2, 3], [1, 2, 3]) == -1
    assert first_difference([1, 2, 3], [1, 5, 3]) == 1
    assert first_difference([1, 2], [1, 2, 3]) == 2
    assert first_difference([], []) == -1
    assert first_difference([], [4]) == 0


def test_faithful_encoder_has_no_findings(vocab, texts):
    ref = _reference(vocab)
    with ShadowVerifier(ref, rate=1.0, encoder=lambda d: _ids(ref(d.numpy().tobytes()))) as sv:
        for t in texts + [b"", b"x"]:
            got = sv.encode(_u8(t))
            assert got.tolist() == ref(t)
        sv.drain()
        st = sv.stats()
    assert st["calls"] == st["sampled"] == st["checked"] == len(texts) + 2
    assert st["mismatches"] == 0 and st["dropped"] == 0 and sv.quarantine == []


@pytest.mark.parametrize("fault", [substitute, delete, shift_split])
def test_planted_fault_is_quarantined(vocab, texts, fault, tmp_path):
    ref = _reference(vocab)
    where = {}

    def faulty(d):
        b = d.numpy().tobytes()
        true = ref(b)
        k = _first_merged(true, len(true) // 2)
        where[b] = k
        return _ids(fault(true, k, vocab))

    qdir = str(tmp_path / "q")
    with ShadowVerifier(ref, rate=1.0, encoder=faulty, quarantine_dir=qdir) as sv:
        outs = [sv.encode(_u8(t)) for t in texts[:3]]
        sv.drain()
        st = sv.stats()
        q = list(sv.quarantine)
    assert st["mismatches"] == 3 and len(q) == 3
    for t, o, s in zip(texts[:3], outs, q):
        assert s.data == t and s.ids == o.tolist() and s.ref_ids == ref(t)
        assert s.first_diff == where[t]
    # offline reproduction from the files
    data, rec = load_sample(os.path.join(qdir, "sample_1"))
    assert data == texts[1]
    assert rec["ref_ids"] == ref(data)
    assert first_difference(rec["ids"], ref(data)) == rec["first_diff"] == where[data]


def test_batch_reports_only_the_faulty_text(vocab, texts):
    ref = _reference(vocab)
    bad_text = 2

    def batch(d, offsets):
        raw = d.numpy().tobytes()
        off = offsets.tolist()
        ids, out_off = [], [0]
        for s in range(len(off) - 1):
            one = ref(raw[off[s]:off[s + 1]])
            if s == bad_text:
                one = delete(one, 5, vocab)
            ids.extend(one)
            out_off.append(len(ids))
        return _ids(ids), torch.tensor(out_off, dtype=torch.int64)

    parts = [texts[0], b"", texts[1], texts[2]]
    raw = b"".join(parts)
    off = torch.tensor(np.cumsum([0] + [len(p) for p in parts]), dtype=torch.int64)
    with ShadowVerifier(ref, rate=1.0, batch_encoder=batch) as sv:
        sv.encode_batch(_u8(raw), off)
        sv.drain()
        st = sv.stats()
    assert st["texts"] == 4 and st["mismatches"] == 1
    (s,) = sv.quarantine
    assert s.text_index == bad_text and s.data == parts[bad_text] and s.first_diff == 5


def test_failing_reference_is_a_finding():
    def broken(b):
        raise ValueError("cannot decode")

    with ShadowVerifier(broken, rate=1.0, encoder=lambda d: _ids(list(d.numpy()))) as sv:
        sv.encode(_u8(b"abc"))
        sv.drain()
    (s,) = sv.quarantine
    assert "ValueError" in s.error and s.ref_ids == []


def test_sampling_fraction():
    n, rate = 20_000, 0.05
    with ShadowVerifier(lambda b: list(b), rate=rate, seed=3, max_pending=n,
                        encoder=lambda d: _ids(list(d.numpy()))) as sv:
        x = _u8(b"ab")
        for _ in range(n):
            sv.encode(x)
        sv.drain()
        st = sv.stats()
    sd = (n * rate * (1 - rate)) ** 0.5
    assert abs(st["sampled"] - n * rate) < 4 * sd
    assert st["checked"] == st["sampled"] and st["mismatches"] == 0


def test_detection_delay_is_geometric():
    """Every call faulty, rate 5 %: the share of verifiers whose first finding
    comes within 42 calls matches 1 - 0.95^42."""
    rate, k, runs, horizon = 0.05, 42, 400, 200
    within = 0
    for seed in range(runs):
        sv = ShadowVerifier(lambda b: list(b), rate=rate, seed=1000 + seed, max_pending=horizon,
                            encoder=lambda d: _ids([0] + list(d.numpy())))
        x = _u8(b"q")
        for _ in range(horizon):
            sv.encode(x)
        sv.close()
        calls = sorted(s.call for s in sv.quarantine)
        assert len(calls) == sv.stats()["sampled"]
        if calls and calls[0] < k:
            within += 1
    p = 1 - (1 - rate) ** k
    assert abs(p - 0.8847) < 1e-3
    sd = (runs * p * (1 - p)) ** 0.5
    assert abs(within - runs * p) < 4 * sd


def test_full_queue_drops_instead_of_blocking():
    release = threading.Event()

    def slow(b):
        release.wait(30)
        return list(b)

    sv = ShadowVerifier(slow, rate=1.0, max_pending=2, encoder=lambda d: _ids(list(d.numpy())))
    x = _u8(b"zz")
    for _ in range(10):
        sv.encode(x)          # must return at once although no check can finish
    st = sv.stats()
    assert st["sampled"] == 10 and 7 <= st["dropped"] <= 8
    release.set()
    sv.close()
    st = sv.stats()
    assert st["checked"] + st["dropped"] == st["sampled"] and st["mismatches"] == 0
    with pytest.raises(RuntimeError):
        sv.encode(x)


def test_rate_zero_checks_nothing():
    with ShadowVerifier(lambda b: [], rate=0.0, encoder=lambda d: _ids(list(d.numpy()))) as sv:
        for _ in range(50):
            sv.encode(_u8(b"abc"))
        sv.drain()
        assert sv.stats()["sampled"] == 0 and sv.quarantine == []
    with pytest.raises(ValueError):
        ShadowVerifier(lambda b: [], rate=1.5)


def test_failing_hook_does_not_stop_the_checks():
    def hook(sample):
        raise OSError("disk full")

    with ShadowVerifier(lambda b: [1], rate=1.0, on_mismatch=hook, encoder=lambda d: _ids([2])) as sv:
        for _ in range(3):
            sv.encode(_u8(b"a"))
        sv.drain()
        st = sv.stats()
    assert st["checked"] == 3 and st["mismatches"] == 3
    assert st["errors"] == 3 and "disk full" in sv.last_error and len(sv.quarantine) == 3
