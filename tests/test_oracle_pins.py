"""Pins of the CPU oracle's primitives against facts outside the oracle:
Python's hashlib (FIPS 180-4 SHA-256), rocRAND's open Philox4x32-10, the
published SplitMix64 output, closed forms of the document hash, and the exact
big-integer form of the hold-out threshold.  No GPU is used."""
import hashlib
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

M64 = (1 << 64) - 1
PHI32 = 0x9E3779B1
PHI64 = 0x9E3779B97F4A7C15
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# --------------------------------------------------------------- SHA-256

@pytest.mark.parametrize("n", [0, 1, 3, 55, 56, 57, 63, 64, 65, 119, 120, 127, 128, 129, 1000, 13 * 64])
def test_sha256_matches_hashlib(n):
    data = bytes((7 * i + 3) & 0xFF for i in range(n))
    assert oracle.sha256(data) == hashlib.sha256(data).digest()


def test_sha256_random_lengths():
    r = np.random.default_rng(5)
    for _ in range(60):
        n = int(r.integers(0, 3000))
        data = r.integers(0, 256, size=n, dtype=np.uint8).tobytes()
        assert oracle.sha256(data) == hashlib.sha256(data).digest()


@pytest.mark.parametrize("T", [1, 3, 17, 60, 64, 100, 4095])
def test_window_digest_is_sha256_of_record(T):
    r = np.random.default_rng(6 + T)
    tok = r.integers(0, 2**32, size=T, dtype=np.uint32)
    pos = r.integers(-5, 100, size=T).astype(np.int32)
    doc = r.integers(-1, 1000, size=T).astype(np.int32)
    mask = r.integers(0, 2, size=T).astype(np.uint8)
    record = (tok.astype("<u4").tobytes() + pos.astype("<i4").tobytes() +
              doc.astype("<i4").tobytes() + mask.tobytes())
    assert len(record) == 13 * T
    assert oracle.window_digest(tok, pos, doc, mask) == hashlib.sha256(record).digest()


def _record(T, seed):
    r = np.random.default_rng(seed)
    tok = r.integers(0, 2**32, size=T, dtype=np.uint32)
    pos = r.integers(-5, 100, size=T).astype(np.int32)
    doc = r.integers(-1, 1000, size=T).astype(np.int32)
    mask = r.integers(0, 2, size=T).astype(np.uint8)
    record = (tok.astype("<u4").tobytes() + pos.astype("<i4").tobytes() +
              doc.astype("<i4").tobytes() + mask.tobytes())
    return tok, pos, doc, mask, record


# one chunk (13·T ≤ 4096), one byte past a chunk, chunks straddling the record's
# arrays, exact multiples of a chunk (T = 1024·k: 13·T = 4096·13k/4) and a long record
@pytest.mark.parametrize("T", [1, 3, 64, 315, 316, 1000, 1024, 2048, 4095, 4096, 5000])
def test_chunked_window_digest_rebuilt_with_hashlib(T):
    """The chunked window digest: SHA-256 of the SHA-256 digests of the record's
    4,096-byte chunks in order, the last chunk shorter."""
    tok, pos, doc, mask, record = _record(T, 70 + T)
    chunks = [record[i:i + 4096] for i in range(0, len(record), 4096)]
    assert sum(map(len, chunks)) == 13 * T and all(len(c) == 4096 for c in chunks[:-1])
    want = hashlib.sha256(b"".join(hashlib.sha256(c).digest() for c in chunks)).digest()
    got = oracle.window_digests_chunked(tok[None], pos[None], doc[None], mask[None])
    assert got.shape == (1, 32) and got[0].tobytes() == want


def test_chunked_window_digest_of_one_chunk_is_double_sha256():
    """A record of at most 4,096 bytes is one chunk: its digest is SHA-256 applied
    twice, and it differs from the whole-record digest."""
    for T in (1, 100, 315):
        tok, pos, doc, mask, record = _record(T, 90 + T)
        got = oracle.window_digests_chunked(tok, pos, doc, mask).tobytes()
        assert got == hashlib.sha256(hashlib.sha256(record).digest()).digest()
        assert got != oracle.window_digest(tok, pos, doc, mask)


def test_chunked_window_digests_batch_layout_and_one_byte():
    """[n, T] windows give [n, 32] digests, window by window; one changed byte in
    any chunk changes that window's digest only."""
    T, n = 700, 5
    rows = [_record(T, 110 + w) for w in range(n)]
    tok, pos, doc, mask = (np.stack([r[k] for r in rows]) for k in range(4))
    d = oracle.window_digests_chunked(tok, pos, doc, mask)
    assert d.shape == (n, 32)
    for w in range(n):
        assert d[w].tobytes() == oracle.window_digests_chunked(tok[w], pos[w], doc[w], mask[w]).tobytes()
    for k, arr in enumerate((tok, pos, doc)):  # chunks 0, 2 and 1 (4·T bytes an array)
        a2 = [tok.copy(), pos.copy(), doc.copy(), mask.copy()]
        a2[k][3, T - 1] ^= 1
        d2 = oracle.window_digests_chunked(*a2)
        assert d2[3].tobytes() != d[3].tobytes()
        assert np.array_equal(np.delete(d2, 3, 0), np.delete(d, 3, 0))


# --------------------------------------------------------------- Philox vs rocRAND

@pytest.fixture(scope="module")
def philox_ref():
    hipcc = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)
    if hipcc is None:
        pytest.skip("hipcc not available to build the rocRAND reference")
    d = tempfile.mkdtemp(prefix="philox_ref_")
    exe = os.path.join(d, "philox_ref")
    subprocess.check_call([hipcc, "-O1", "-o", exe, os.path.join(ROOT, "tests", "pins", "philox_rocrand.cpp")],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)

    def run(rows):
        text = "\n".join(" ".join("%x" % v for v in row) for row in rows) + "\n"
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [[int(x, 16) for x in line.split()] for line in out.strip().splitlines()]

    yield run
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_rocrand(philox_ref):
    r = np.random.default_rng(11)
    rows = [[0] * 6, [0xFFFFFFFF] * 6, [1, 0, 0x53485546, 0, 0, 0]]
    rows += r.integers(0, 2**32, size=(300, 6), dtype=np.uint64).tolist()
    ref = philox_ref(rows)
    for row, want in zip(rows, ref):
        got = oracle.philox4x32_10(row[:4], row[4:]).tolist()
        assert got == want, row


def test_shuffle_key_layout(philox_ref):
    r = np.random.default_rng(12)
    seeds = [0, 1, 2**63 + 5] + r.integers(0, 2**63, size=20).tolist()
    docs = [0, 1, 2**32 - 1, 2**32, 2**40 + 7] + r.integers(0, 2**31, size=20).tolist()
    rows = [[d & 0xFFFFFFFF, d >> 32, 0x53485546, 0, s & 0xFFFFFFFF, s >> 32] for s in seeds for d in docs]
    ref = philox_ref(rows)
    for row, want in zip(rows, ref):
        seed = row[4] | (row[5] << 32)
        d = row[0] | (row[1] << 32)
        assert oracle.shuffle_key(seed, d) == (want[1] << 32) | want[0]


# --------------------------------------------------------------- mix64 (SplitMix64 output function)

def test_mix64_published_splitmix64_value():
    # SplitMix64 (Steele, Lea & Flood 2014) from state 0 adds the golden gamma
    # and applies the output function; its first output is 0xE220A8397B1DCDAF.
    assert oracle.mix64(PHI64) == 0xE220A8397B1DCDAF


def _unxorshift(y, k):
    x = y
    for _ in range(64 // k + 1):
        x = y ^ (x >> k)
    return x & M64


def test_mix64_inverts():
    # The output function is a bijection; undo it with modular inverses of the
    # two multipliers (computed here by Python, not taken from the oracle).
    m1, m2 = 0xBF58476D1CE4E5B9, 0x94D049BB133111EB
    i1, i2 = pow(m1, -1, 1 << 64), pow(m2, -1, 1 << 64)
    r = np.random.default_rng(13)
    for x in [0, 1, M64] + r.integers(0, 2**63, size=200).tolist():
        y = oracle.mix64(x)
        z = _unxorshift(y, 31)
        z = (z * i2) & M64
        z = _unxorshift(z, 27)
        z = (z * i1) & M64
        z = _unxorshift(z, 30)
        assert z == x
    assert oracle.mix64(0) == 0


# --------------------------------------------------------------- document hash: closed forms

def _k(i):
    return ((i + 1) * PHI32) & 0xFFFFFFFF


def test_hash_of_empty_document_is_zero():
    assert oracle.doc_hash(np.zeros(0, np.uint32)) == 0


@pytest.mark.parametrize("L", [1, 2, 3, 8, 9, 257, 1000, 4097])
def test_hash_with_cancelled_keys(L):
    # t_i = -k_i makes every even-position factor zero, so S = 0.
    t = np.array([(-_k(i)) & 0xFFFFFFFF for i in range(L)], dtype=np.uint32)
    assert oracle.doc_hash(t) == oracle.mix64((L * PHI64) & M64)


@pytest.mark.parametrize("L", [1, 2, 5, 64, 65, 999])
def test_hash_with_unit_factors(L):
    # t_i = 1 - k_i makes every factor 1; an odd length's last pair is 1·k_L.
    t = np.array([(1 - _k(i)) & 0xFFFFFFFF for i in range(L)], dtype=np.uint32)
    S = L // 2 if L % 2 == 0 else (L - 1) // 2 + _k(L)
    assert oracle.doc_hash(t) == oracle.mix64((S ^ (L * PHI64)) & M64)


def test_hash_as_sum_of_chosen_products():
    # With t_i = x_i - k_i the pair factors are the x_i, so
    # S = Σ x_{2j}·x_{2j+1} mod 2^64 for any chosen x: this fixes the pairing,
    # the key of every position and the 64-bit accumulation.
    r = np.random.default_rng(14)
    for L in [2, 3, 10, 11, 100, 101, 4096, 5001]:
        x = r.integers(0, 2**32, size=L + 1, dtype=np.uint64).tolist()
        if L % 2:
            x[L] = _k(L)  # the virtual token 0 contributes its key as factor
        t = np.array([(x[i] - _k(i)) & 0xFFFFFFFF for i in range(L)], dtype=np.uint32)
        S = sum(x[2 * j] * x[2 * j + 1] for j in range((L + 1) // 2)) & M64
        assert oracle.doc_hash(t) == oracle.mix64(S ^ ((L * PHI64) & M64))


# --------------------------------------------------------------- hold-out threshold

@pytest.mark.parametrize("bp", [0, 1, 100, 500, 9999, 10000])
def test_held_threshold_is_exact(bp):
    # held ⇔ floor(h·10000/2^64) < bp ⇔ h < ceil(bp·2^64/10000)
    edge = -((-bp << 64) // 10000)
    if edge > 0:
        assert oracle.held(edge - 1, bp)
    if edge <= M64:
        assert not oracle.held(edge, bp)
    r = np.random.default_rng(bp)
    for h in r.integers(0, 2**63, size=200).tolist() + [0, M64]:
        assert oracle.held(h, bp) == (((h * 10000) >> 64) < bp)


def test_holdout_rate_within_four_sigma():
    from synth import make_corpus
    c = make_corpus("pretrain", 0.03)
    p = oracle.Plan(c)
    n = np.bincount(c.source.astype(np.int64), minlength=c.n_sources)
    for s in range(c.n_sources):
        q = c.holdout_bp[s] / 1e4
        mu, sd = n[s] * q, (n[s] * q * (1 - q)) ** 0.5
        assert abs(int(p.held_docs[s]) - mu) <= 4 * sd + 1, (s, p.held_docs[s], mu, sd)


def test_batch_with_chunked_digests():
    """With digest_chunked the oracle's batches keep every array and learned count,
    and each window digest is the hashlib rebuild of its record's chunks."""
    from synth.corpus import random_small
    c = random_small(7, n_docs=300, n_sources=2, T=400, B=3, max_len=900)
    a = oracle.Plan(c)
    a.cycle(0)
    b = oracle.Plan(c.replace(digest_chunked=True))
    b.cycle(0)
    x, y = a.batch(0, 2), b.batch(0, 2)
    for k in ("tokens", "pos", "doc", "mask", "learned"):
        assert np.array_equal(x[k], y[k]), k
    for s in range(2):
        for w in range(3):
            rec = (y["tokens"][s, w].astype("<u4").tobytes() + y["pos"][s, w].astype("<i4").tobytes() +
                   y["doc"][s, w].astype("<i4").tobytes() + y["mask"][s, w].tobytes())
            inner = b"".join(hashlib.sha256(rec[i:i + 4096]).digest() for i in range(0, len(rec), 4096))
            assert y["digests"][s, w].tobytes() == hashlib.sha256(inner).digest()
            assert x["digests"][s, w].tobytes() == hashlib.sha256(rec).digest()
