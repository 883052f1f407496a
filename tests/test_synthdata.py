"""Input generators: determinism, event layout, bf16 rounding."""
import numpy as np
import torch

from synthdata import bf16_round, bf16_bits, event_bytes, gen_hnet_tiny, gen_event_streams, gen_coding_rate_fp32, cluster_rows


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 10000),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_round(x), want)
    assert bf16_bits(np.array([1.0], np.float32))[0] == 0x3F80


def test_generators_are_deterministic():
    a, b = gen_event_streams(nseq=3, d=16, max_events=40), gen_event_streams(nseq=3, d=16, max_events=40)
    assert np.array_equal(a["bytes"], b["bytes"]) and np.array_equal(a["q"], b["q"])
    assert np.array_equal(gen_hnet_tiny()["q"], gen_hnet_tiny()["q"])
    assert np.array_equal(gen_coding_rate_fp32(nseq=1, T=64, d=16)["h"], gen_coding_rate_fp32(nseq=1, T=64, d=16)["h"])


def test_event_layout():
    rng = np.random.default_rng(1)
    n = 500
    ev = event_bytes(rng, n).reshape(n, 32)
    words = ev.view("<u8").reshape(n, 4)
    typ = ev[:, 0]
    assert set(np.unique(typ)) <= {0, 1, 2, 3}
    assert np.all(ev[:, 28:] == 0)
    ts = words[:, 1]
    assert np.all(np.diff(ts.astype(np.float64)) > 0)
    price = words[:, 2].view(np.int64)
    assert np.all(np.abs(np.diff(price)) == 1)
    qty = ev[:, 24:28].copy().view("<u4").reshape(-1)
    assert np.all(qty >= 1)
    gaps = np.diff(ts.astype(np.float64))
    assert 0.15e6 < np.median(gaps) < 0.45e6  # Pareto(1.5) median 0.271 ms


def test_c1_offsets_and_ragged_lengths():
    c = gen_event_streams(nseq=6, d=8)
    L = np.diff(c["offsets"])
    assert np.all(L % 32 == 0) and np.all((L >= 32 * 32) & (L <= 32 * 256))
    assert c["h"].shape == (c["offsets"][-1], 8)


def test_cluster_rows_unit_norm():
    h = cluster_rows(np.random.default_rng(2), 2, 100, 16)
    np.testing.assert_allclose(np.linalg.norm(h, axis=2), 1.0, rtol=1e-12)
