"""Pins of the oracle's padding-free rows (Linnet Training, Supervised
fine-tuning, the transformers Trainer path: the padding is removed, the rows
are packed into one sequence whose length rounds up to a multiple of 256, and
a position id 0 starts each sequence).  Checked against the padded batch the
same plan emits: the packed row is exactly the concatenation of each window's
non-padding prefix, in slot order."""
import numpy as np
import pytest

import oracle
from synth import make_corpus, random_small


@pytest.mark.parametrize("seed,bucket,world", [(s, b, w) for s in range(4) for b in (256, 64, 1) for w in (1, 2)])
def test_packed_row_is_the_padded_batch_without_padding(seed, bucket, world):
    c = random_small(1300 + seed, n_docs=200, n_sources=2, T=64, B=4, max_len=90, prompts=bool(seed % 2))
    p = oracle.Plan(c)
    info = p.cycle(0)
    n = min(3, info.n_updates)
    padded = p.batch(0, n, world=world, digests=False)
    packed = p.batch_packed(0, n, world=world, bucket=bucket)
    per, T = c.B // world, c.T
    for i in range(n):
        parts = {k: [] for k in ("tokens", "pos", "doc", "mask")}
        starts = [0]
        for jj in range(per):
            real = int((padded["doc"][i, jj] >= 0).sum())
            for k in parts:
                parts[k].append(padded[k][i, jj, :real])
            starts.append(starts[-1] + real)
        assert packed["row_start"][i].tolist() == starts
        total = starts[-1]
        L = total if bucket <= 1 else -(-total // bucket) * bucket
        L = min(L, per * T)
        assert int(packed["length"][i]) == L and L % max(bucket, 1) == 0 or L == per * T
        for k in parts:
            cat = np.concatenate(parts[k])
            assert np.array_equal(packed[k][i, :total], cat), (i, k)
        # padding between the total and the length
        assert (packed["doc"][i, total:L] == -1).all() and (packed["pos"][i, total:L] == 0).all()
        assert (packed["mask"][i, total:L] == 0).all() and (packed["tokens"][i, total:L] == c.pad_token).all()
        # a position id 0 starts every sequence: each window's first position, and each piece's
        for jj in range(per):
            if starts[jj + 1] > starts[jj]:
                assert packed["pos"][i, starts[jj]] == 0


def test_packed_learned_positions_match_the_padded_mask():
    c = make_corpus("sft", 0.001)
    p = oracle.Plan(c)
    p.cycle(0)
    padded = p.batch(0, 2, digests=False)
    packed = p.batch_packed(0, 2)
    for i in range(2):
        assert int(packed["mask"][i].sum()) == int(padded["mask"][i].sum()) == int(padded["learned"][i])
