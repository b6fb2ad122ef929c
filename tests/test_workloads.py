"""The seeded generators produce the shapes and structure they promise."""
import math

import numpy as np
import torch

from workloads import (bf16_bits_to_f32, config, draw_unit, f32_to_bf16_bits, make_workload, scaled,
                       storage_to_f64)


def test_bf16_rounding_matches_torch():
    """Round-to-nearest-even to bf16, checked against torch's conversion."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8], dtype=np.float32)])
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_unit_independent():
    s = scaled(3, "B")
    w1 = make_workload(s, threads=4)
    w2 = make_workload(s, threads=1)
    np.testing.assert_array_equal(w1.k, w2.k)
    np.testing.assert_array_equal(w1.block_table, w2.block_table)
    q, K, V = draw_unit(s, 1, 1, int(w1.context_lens[1]))
    np.testing.assert_array_equal(w1.q[1, 4:8], q)


def test_paged_structure_and_poison():
    w = make_workload(scaled(3, "A"))
    P = w.spec.page_size
    n_pages = (w.context_lens + P - 1) // P
    used = np.concatenate([w.block_table[b, :n_pages[b]] for b in range(w.spec.batch)])
    assert len(np.unique(used)) == len(used) == n_pages.sum()           # a permutation of the pool
    poison = w.k.shape[0] - 1
    assert np.all(np.isnan(storage_to_f64(w.k[poison], "bf16")))
    for b in range(w.spec.batch):
        assert np.all(w.block_table[b, n_pages[b]:] == poison)
        n = int(w.context_lens[b])
        if n % P:
            last = w.block_table[b, n_pages[b] - 1]
            assert np.all(np.isnan(storage_to_f64(w.v[last, :, n % P:], "bf16")))


def test_reading_b_logit_shifts():
    """Mean-query scores move by +6 at the sinks and by 3*exp(-dist/2048) for
    recency, up to the unit-variance key noise; 1% of values are scaled by 8."""
    s = config(2, "B", batch=1, num_q_heads=4, num_kv_heads=1, ctx=(8192, 8192))
    q, K, V = draw_unit(s, 0, 0, 8192)
    qf = storage_to_f64(q, "bf16")
    qbar = qf.mean(0)
    sc = storage_to_f64(K, "bf16") @ qbar / math.sqrt(128)
    noise = np.linalg.norm(qbar) / math.sqrt(128)         # std of the noise part
    assert abs(sc[:4].mean() - (6 + 3 * np.exp(-8191 / 2048))) < 3 * noise
    assert abs(sc[-64:].mean() - 3 * np.exp(-np.arange(63, -1, -1) / 2048).mean()) < 1.0 * noise
    vn = np.linalg.norm(storage_to_f64(V, "bf16"), axis=1)
    assert (vn > 4 * math.sqrt(128)).sum() == 8192 // 100


def test_kept_list_rules():
    w = make_workload(scaled(5, "B"))
    T = int(w.num_blocks[0])
    for b in range(w.spec.batch):
        for h in range(w.spec.num_kv_heads):
            lst = w.kept_blocks[b, h, : w.kept_count[b, h]]
            assert len(lst) == math.ceil(0.5 * T)
            assert np.all(np.diff(lst) > 0) and lst[0] == 0
            assert set(range(T - w.spec.kept_recent, T)) <= set(lst.tolist())


def test_full_config_shapes():
    c3 = config(3)
    assert (c3.batch, c3.num_q_heads, c3.num_kv_heads, c3.head_dim, c3.page_size) == (64, 32, 8, 128, 16)
    assert config(5).kept_frac == 0.5 and config(1).dtype == "f32"
