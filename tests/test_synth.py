import numpy as np

from sparse_kv_cache_amd import synth


def test_deterministic_and_streaming_matches():
    k1, q1 = synth.make_inputs(3, 2, 500, 8)
    k2, q2 = synth.make_inputs(3, 2, 500, 8)
    assert k1.tobytes() == k2.tobytes() and q1.tobytes() == q2.tobytes()
    parts = list(synth.stream_inputs(3, 2, 500, 8))
    assert np.array_equal(parts[0][2], k1[0]) and np.array_equal(parts[1][2], k1[1])
    assert np.array_equal(parts[2][1], q1)
    k3, _ = synth.make_inputs(4, 2, 500, 8)
    assert not np.array_equal(k1, k3)


def test_distribution_shape():
    keys, q = synth.make_inputs(0, 1, 20000, 4)
    assert keys.dtype == np.float32 and q.dtype == np.float32
    # the recipe: log-normal channel scales, four of them multiplied by 8
    rng = np.random.default_rng(0)
    sigma = rng.lognormal(0.0, 0.5, 128).astype(np.float32)
    outl = rng.choice(128, 4, replace=False)
    sigma[outl] *= np.float32(8)
    sd = keys[0].std(axis=0)
    assert np.allclose(sd, sigma, rtol=0.05)
    assert np.abs(q).max() < 8


def test_workload_table():
    w = synth.WORKLOADS["qwen3_8b_1m"]
    assert (w.num_kv_heads, w.n, w.group, w.k, w.num_q) == (8, 1 << 20, 4, 2048, 32)
    assert synth.WORKLOADS["multi_session"].num_q == 512


def test_planted_keys_have_the_requested_logit():
    keys, q = synth.make_inputs(5, 1, 5000, 3)
    k = keys[0].copy()
    rows = synth.plant_aligned_keys(5, k, q, 16, 12.0)
    assert rows.shape == (3, 16) and len(np.unique(rows)) == 48
    for g in range(3):
        logits = k[rows[g]].astype(np.float64) @ q[g].astype(np.float64) / np.sqrt(128)
        assert np.all(np.abs(logits - 12.0) < 0.1 * np.linalg.norm(q[g]) / np.sqrt(128) * 5)
    untouched = np.setdiff1d(np.arange(5000), rows.ravel())
    assert np.array_equal(k[untouched], keys[0][untouched])
