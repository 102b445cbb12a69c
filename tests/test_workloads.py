"""The seeded generator: determinism, shapes, bf16 rounding and the embedding recipe."""
import numpy as np
import torch

from workloads import WORKLOADS, custom_workload, head_gains, make_embedding, make_inputs


def test_named_workload_shapes():
    w = WORKLOADS["video-32k"]
    assert (w.seq_len, w.heads, w.head_dim, w.block, w.num_blocks, w.units) == (32760, 40, 128, 64, 512, 20480)
    assert w.grid[0] * w.grid[1] * w.grid[2] == w.seq_len
    w5 = WORKLOADS["video-119k"]
    assert (w5.num_blocks, w5.seq_len - (w5.num_blocks - 1) * w5.block) == (929, 16)
    assert w5.grid[0] * w5.grid[1] * w5.grid[2] == w5.seq_len


def test_inputs_deterministic_and_dtype():
    w = custom_workload(1, 3, 300, 64, 64, dtype="bf16", top_p=0.9)
    a = make_inputs(w, seed=0, threads=1)
    b = make_inputs(w, seed=0, threads=4)
    c = make_inputs(w, seed=1, threads=2)
    for x, y, z in zip(a, b, c):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 3, 300, 64) and x.is_contiguous()
        assert torch.equal(x, y)
        assert not torch.equal(x, z)


def test_bf16_is_round_to_nearest_even_of_fp32_draws():
    w = custom_workload(1, 1, 64, 64, 64, dtype="bf16", structured=False, wid=7)
    q, _, _ = make_inputs(w, seed=3, threads=1)
    z = np.random.Generator(np.random.PCG64(np.random.SeedSequence([3, 7, 0, 0, 0]))).standard_normal(
        (64, 64), dtype=np.float32)
    bits = z.view(np.uint32).astype(np.uint64)
    rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    got = q[0, 0].view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, rne)


def test_embedding_rms_and_gain_ranges():
    w = WORKLOADS["skewed-32k"]
    e = make_embedding(w)
    assert e.shape == (w.seq_len, w.head_dim)
    np.testing.assert_allclose(np.sqrt((e.astype(np.float64) ** 2).mean(1)), w.embed_rms, rtol=1e-5)
    g = head_gains(w)
    assert g.shape == (40,) and g.min() >= 0.25 and g.max() <= 8.0
    g3 = head_gains(WORKLOADS["video-32k"])
    assert g3.min() >= 0.5 and g3.max() <= 4.0
