"""GPU check of spec_verify_check_inputs: violations planted in otherwise
valid inputs are counted exactly; the expected counts are the checks'
definitions written out in numpy."""
import numpy as np
import pytest
import torch

import speculative_decoding_verify_attn_amd as sv

pytestmark = pytest.mark.gpu


def _expected(table, lens, T, num_blocks, tokens, V, uniforms):
    maxb = table.shape[1]
    c = np.zeros(4, dtype=np.int64)
    c[0] = int(np.sum((lens < T) | (lens > 16 * maxb)))
    for b, L in enumerate(lens):
        np_b = (min(max(int(L), 0), 16 * maxb) + 15) // 16
        e = table[b, :np_b]
        c[1] += int(np.sum((e < 0) | (e >= num_blocks)))
    c[2] = int(np.sum((tokens < 0) | (tokens >= V)))
    c[3] = int(np.sum(~((uniforms >= 0) & (uniforms < 1))))
    return c


def _inputs(seed, B, maxb, num_blocks, K, V):
    rng = np.random.default_rng(seed)
    T = K + 1
    lens = rng.integers(T, 16 * maxb + 1, size=B).astype(np.int32)
    table = rng.integers(0, num_blocks, size=(B, maxb)).astype(np.int32)
    tokens = rng.integers(0, V, size=(B, K)).astype(np.int32)
    uniforms = rng.random((B, K + 1)).astype(np.float32)
    return T, lens, table, tokens, uniforms


def _run(B, T, lens, table, num_blocks, toks, V, us, **skip):
    dev = torch.device("cuda", 0)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    args = dict(block_table=t(table), context_lens=t(lens), tokens=t(toks), uniforms=t(us))
    args.update(skip)
    counts = sv.spec_verify_check_inputs(B, T=T, max_blocks_per_seq=table.shape[1], num_blocks=num_blocks, V=V, **args)
    torch.cuda.synchronize()
    return counts.cpu().numpy().astype(np.int64)


def test_clean_inputs_count_nothing():
    B, maxb, nb, K, V = 37, 300, 5000, 5, 128256
    T, lens, table, tokens, u = _inputs(1, B, maxb, nb, K, V)
    assert list(_run(B, T, lens, table, nb, tokens, V, u)) == [0, 0, 0, 0]


def test_planted_violations_are_counted():
    B, maxb, nb, K, V = 41, 700, 9000, 7, 32000   # 700 pages: a sequence's check loops over its pages
    T, lens, table, tokens, u = _inputs(2, B, maxb, nb, K, V)
    rng = np.random.default_rng(3)
    lens[[0, 5, 9]] = [T - 1, 16 * maxb + 1, -4]
    lens[[1, 2]] = [16 * maxb, T]                     # the bounds themselves are valid
    lens[[3, 4, 6]] = 100                             # 7 visible pages each
    for b in (3, 4, 6):
        np_b = (int(lens[b]) + 15) // 16
        table[b, rng.choice(np_b, size=3, replace=False)] = [-1, nb, 2 ** 30]
        if np_b < maxb:
            table[b, np_b:] = -7                      # past the visible pages: not counted
    tokens[7, 0], tokens[8, K - 1], tokens[10, 3] = -1, V, 2 ** 31 - 1
    u[11, 0], u[12, K], u[13, 2], u[14, 1], u[15, 4] = 1.0, -1e-7, np.nan, np.inf, 0.0   # 0.0 is valid
    want = _expected(table, lens, T, nb, tokens, V, u)
    assert want[0] == 3 and want[1] == 9 and want[2] == 3 and want[3] == 4
    got = _run(B, T, lens, table, nb, tokens, V, u)
    assert list(got) == list(want)
    # a second call clears the counters first
    assert list(_run(B, T, lens, table, nb, tokens, V, u)) == list(want)


def test_skipped_checks():
    B, maxb, nb, K, V = 9, 40, 300, 4, 1000
    T, lens, table, tokens, u = _inputs(4, B, maxb, nb, K, V)
    lens[0] = 0
    tokens[1, 1] = V
    u[2, 0] = 2.0
    got = _run(B, T, lens, table, nb, tokens, V, u, block_table=None, uniforms=None)
    assert list(got) == [1, 0, 1, 0]
    got = _run(B, T, lens, table, nb, tokens, V, u, context_lens=None, block_table=None, tokens=None)
    assert list(got) == [0, 0, 0, 1]
