"""The seeded input generator and the synthetic length mix."""
import os

import numpy as np
import torch

import dcp_inputs as di

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_sequence():
    # splitmix64 seeded with 0 (Steele, Lea & Flood 2014; public-domain reference code)
    out = [int(x) for x in di.splitmix64_at(0, np.arange(3))]
    assert out == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(200000).astype(np.float32) * 7
    ours = di.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_compiled_host_generator_matches_numpy():
    rows = np.random.default_rng(2).integers(0, 2 ** 40, size=700).astype(np.uint64)
    for cols in (576, 128, 7):
        assert np.array_equal(di.host_rows(rows, cols, 5, 1), di.host_rows_numpy(rows, cols, 5, 1))
    assert np.array_equal(di.host_rows(rows, 40, 0, 0, mode=1), di.census_rows_numpy(rows, 40))


def test_float64_host_generator_is_the_widened_bf16_one():
    rows = np.random.default_rng(3).integers(0, 2 ** 40, size=900).astype(np.uint64)
    for cols, mode in ((576, 0), (128, 0), (40, 1)):
        wide = di.host_rows_f64(rows, cols, 6, 2, mode=mode)
        assert wide.dtype == np.float64
        assert np.array_equal(wide, di.bf16_bits_to_f64(di.host_rows(rows, cols, 6, 2, mode=mode)))
    t = np.array([0, 5, 77, 1 << 20])
    assert np.array_equal(di.host_latent_f64(3, t, 576, 4), di.bf16_bits_to_f64(di.host_latent(3, t, 576, 4)))
    assert np.array_equal(di.host_gqa_kv_f64(2, t, 4, 128, 4, di.STREAM_V),
                          di.bf16_bits_to_f64(di.host_gqa_kv(2, t, 4, 128, 4, di.STREAM_V)))


def test_generator_statistics_and_independence():
    z = di.bf16_bits_to_f64(di.host_rows(np.arange(4000, dtype=np.uint64), 576, 1, 1))
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1.0) < 0.01 and np.abs(z).max() <= 6.0
    a = di.host_rows(np.arange(10, dtype=np.uint64), 64, 1, di.STREAM_K)
    b = di.host_rows(np.arange(10, dtype=np.uint64), 64, 1, di.STREAM_V)
    c = di.host_rows(np.arange(10, dtype=np.uint64), 64, 2, di.STREAM_K)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_length_mix_matches_pages():
    target = {}
    with open(os.path.join(GOLDEN, "workload_length_mix.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v, tol = line.split()
                target[k] = (float(v), float(tol))
    for B, seed in [(512, 4), (128, 3)]:
        L = di.bimodal_lengths(B, seed)
        got = {
            "median_tokens": float(np.median(L)),
            "frac_ge_64k": float((L >= 65536).mean()),
            "frac_lt_64k": float((L < 65536).mean()),
            "frac_lt_8k": float((L < 8192).mean()),
            "frac_gt_128k": float((L > 131072).mean()),
            "frac_gt_256k": float((L > 262144).mean()),
        }
        for k, v in got.items():
            assert abs(v - target[k][0]) <= target[k][1], (B, k, v)
        assert L.max() <= target["max_tokens_at_most"][0]
        assert L.max() >= target["max_tokens_at_least"][0]
        assert L.min() >= 1024


def test_workload_shapes():
    w = di.WORKLOADS
    assert w["mla_tiny"].lengths == (1000, 3000)
    g = np.asarray(w["gqa_b32"].lengths)
    assert g.size == 32 and g.min() >= 4096 and g.max() <= 32768
    assert w["mla_1m"].lengths == (1048576,)
    assert len(w["mla_long_b128"].lengths) == 128 and len(w["mla_c512"].lengths) == 512


def test_band_lengths_stay_in_band():
    """Band draws come from the synthetic mix restricted to the band: every length is
    inside it, and the draws follow the mix's quantiles there (a band that the mix covers
    uniformly gets a near-uniform spread)."""
    import dcp_inputs as di
    for lo, hi in di.LENGTH_BANDS:
        L = di.band_lengths(lo, hi, 200, seed=3)
        assert L.min() >= max(lo, 1024) and L.max() < min(hi, di.MAX_SEQ_LEN + 1)
    # 32k..64k lies inside the mix's uniform segment [8192, 65536): stratified draws are
    # evenly spaced there
    L = np.sort(di.band_lengths(32768, 65536, 64, seed=3))
    assert abs(np.median(L) - 49152) < 600 and np.all(np.diff(L) > 0)
    w = di.band_workload(65536, 131072)
    assert abs(sum(w.lengths) / 8 - 1.25e6) < 0.02e6
