"""Synthetic input generators: bf16 rounding, determinism, workload structure."""
import numpy as np
import torch

from block_sparse_flashattention_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-5, 5, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_seeded():
    w = inputs.scaled(inputs.WORKLOADS["gqa_planted_16k"], N=512, Hq=4, Hkv=2)
    a = inputs.generate(w, 0)
    b = inputs.generate(w, 0)
    c = inputs.generate(w, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    # one KV group alone gives the same tensors as the whole workload
    qg, kg, vg = inputs.generate_group(w, 0, 0, 1)
    assert np.array_equal(qg, a[0][0, 2:4]) and np.array_equal(kg, a[1][0, 1])


def test_planted_blocks_shift_keys():
    w = inputs.scaled(inputs.WORKLOADS["gqa_planted_16k"], N=4096, Hq=2, Hkv=1)
    q, k, v = inputs.generate(w, 0)
    kf = inputs.bits_to_f32(k[0, 0]).reshape(64, 64, w.d)
    u = inputs._unit((inputs.STRUCTURE_SEED, inputs.SID_U, 0), w.d)
    proj = (kf @ u).mean(axis=1)  # mean projection per 64-token block
    planted = proj > 1.0
    assert planted.sum() == round(0.10 * 64)
    assert np.all(np.abs(proj[~planted]) < 0.5)


def test_sink_local_structure():
    w = inputs.scaled(inputs.WORKLOADS["sink_local_64k"], N=1024, Hq=2, Hkv=1)
    q, k, v = inputs.generate(w, 0)
    qf = inputs.bits_to_f32(q[0]).astype(np.float64)
    kf = inputs.bits_to_f32(k[0, 0]).astype(np.float64)
    s = qf[0] @ kf.T / np.sqrt(w.d)
    near = np.mean([s[i, i - 1] for i in range(200, 1024)])
    far = np.mean([s[i, i - 500] for i in range(600, 1024)])
    assert near > far + 0.2  # the rotation bias decays with distance
    assert s[:, 0].mean() > s[:, 1:].mean() + 0.7  # key 0 is a sink
