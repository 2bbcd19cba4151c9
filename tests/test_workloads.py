"""The seeded input generator: determinism, row addressing and bf16 rounding."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(3)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -2.5, 3.00390625, 1.00390625, 1.01171875, 65504.0, 1e-30], np.float32)])
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_draw_deterministic_and_row_addressable():
    full = workloads.draw(5, workloads.TENSOR_K, 1, 2, 3000, 16, 0.5, "f32")
    again = workloads.draw(5, workloads.TENSOR_K, 1, 2, 3000, 16, 0.5, "f32")
    assert np.array_equal(full, again)
    pos = np.array([2999, 0, 1024, 1500, 7])
    sub = workloads.draw(5, workloads.TENSOR_K, 1, 2, 3000, 16, 0.5, "f32", positions=pos)
    assert np.array_equal(sub, full[:, :, pos])
    other = workloads.draw(5, workloads.TENSOR_V, 1, 2, 3000, 16, 0.5, "f32")
    assert not np.array_equal(other, full)
    bf = workloads.draw(5, workloads.TENSOR_K, 1, 2, 3000, 16, 0.5, "bf16")
    assert bf.dtype == np.uint16 and np.array_equal(bf, workloads.f32_to_bf16_bits(full))


def test_sample_rows_cover_chunk_edges():
    rows = workloads.sample_rows(8192, 4096, 248, 1)
    for r in (0, 1, 2, 3, 4092, 4093, 4094, 4095, 4096, 4099, 8188, 8191):
        assert r in rows
    assert rows.min() >= 0 and rows.max() < 8192 and np.all(np.diff(rows) > 0)
