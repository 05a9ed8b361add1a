"""The seeded generator: determinism and the statistics the configs promise."""

import numpy as np

import dgq_data


def test_deterministic_and_independent_streams():
    cfg = dgq_data.get_config(2, seq_len=512, batch=2)
    a = dgq_data.head_kv(cfg, 0, 0, 1, 3, 512)
    b = dgq_data.head_kv(cfg, 0, 0, 1, 3, 512)
    c = dgq_data.head_kv(cfg, 0, 0, 1, 4, 512)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0])


def test_batch_layout_matches_heads():
    cfg = dgq_data.get_config(4, batch=3, seq_len=300, min_len=100)
    k, v, cu, lens = dgq_data.batch_kv(cfg, 0)
    assert k.shape == (int(cu[-1]), cfg.hkv, cfg.head_dim) and k.dtype == np.float16
    for b in range(3):
        assert 100 <= lens[b] <= 300
        kk, vv = dgq_data.head_kv(cfg, 0, 0, b, 5, int(lens[b]))
        assert np.array_equal(k[cu[b]:cu[b + 1], 5], kk)
        assert np.array_equal(v[cu[b]:cu[b + 1], 5], vv)


def test_sigma_profiles():
    for cid in (1, 2, 3, 5):
        cfg = dgq_data.get_config(cid)
        length = min(cfg.seq_len, 4096)
        for h in range(4):
            sig, cuts, sigs = dgq_data.head_profile(cfg, 0, 0, 0, h % cfg.hkv, length)
            edges = np.concatenate([[0], cuts, [cfg.total_len(length)]])
            assert np.all(np.diff(edges) >= 32)
            assert len(sigs) in cfg.nseg_choices
            assert np.all((sigs >= 0.03) & (sigs <= 0.47))
    tiny = dgq_data.get_config(1)
    _, _, sigs = dgq_data.head_profile(tiny, 0, 0, 0, 0, 256)
    assert sorted(sigs) == [0.03, 0.15, 0.47]


def test_outliers_at_eight_sigma():
    cfg = dgq_data.get_config(3, seq_len=4096)
    k, _ = dgq_data.head_kv(cfg, 0, 0, 0, 0, 4096)
    sig, _, _ = dgq_data.head_profile(cfg, 0, 0, 0, 0, 4096)
    ratio = np.abs(k.astype(np.float32)) / sig[:, None]
    frac = np.mean(np.abs(ratio - 8.0) < 0.01)
    assert 0.007 < frac < 0.013


def test_block_tables():
    cfg = dgq_data.get_config(2, batch=4, seq_len=100)
    table, n = dgq_data.block_tables(cfg, 0)
    assert n == 4 * 7 and table.shape == (4, 7)
    assert sorted(table.reshape(-1).tolist()) == list(range(n))
    seq = dgq_data.get_config(1)
    table, n = dgq_data.block_tables(seq, 0)
    assert table.tolist() == [list(range(16))]
    stream = dgq_data.get_config(5, batch=2)
    table, n = dgq_data.block_tables(stream, 0)
    assert table.shape == (2, 36)
