"""The seeded input generators: determinism, shapes and the ragged workload's
fixed draw (lengths first, then the page permutation)."""
import numpy as np

from mla_latent_kv_22_amd import inputs as I


def test_deterministic_and_seed_sensitive():
    cfg = I.scaled(I.V2LITE, batch=2, seq_len=130)
    a, b = I.make(cfg, 0), I.make(cfg, 0)
    assert I.digest(a) == I.digest(b)
    assert I.digest(I.make(cfg, 1)) != I.digest(a)


def test_chunked_draws_match_one_draw():
    rng1 = np.random.default_rng(7)
    x = I._normal(rng1, (5000,), 0.5, "bf16", chunk=777)
    rng2 = np.random.default_rng(7)
    y = I._normal(rng2, (5000,), 0.5, "bf16", chunk=1 << 20)
    assert np.array_equal(x, y)


def test_ragged_lengths_and_pages():
    rng = np.random.default_rng(0)
    lens = I.seq_lengths(I.RAGGED, rng)
    assert lens.shape == (128,) and lens.min() >= 512 and lens.max() <= 32768
    assert int(lens.sum()) == 2174306
    assert int(((lens.astype(np.int64) + 63) // 64).sum()) == 34043
    # algorithmic latent-cache bytes of one decode pass
    assert int(lens.sum()) * 576 * 2 == 2504800512


def test_block_table_is_page_permutation():
    cfg = I.scaled(I.RAGGED, batch=6, seq_len=700, min_seq_len=65)
    d = I.make(cfg, 3)
    lens, bt = d["seq_lens"], d["block_table"]
    used = []
    for b in range(cfg.batch):
        n = (int(lens[b]) + 63) // 64
        used += bt[b, :n].tolist()
    assert sorted(used) == list(range(d["num_pages"]))
    # decode: the new token of sequence b goes to position len-1 in its last page
    for b in range(cfg.batch):
        p = int(lens[b]) - 1
        assert d["positions"][b] == p
        assert d["slots"][b] == int(bt[b, p // 64]) * 64 + p % 64


def test_full_path_shapes():
    d = I.make(I.TINY, 0)
    assert d["h"].shape == (512, 256) and d["h"].dtype == np.float32
    assert d["w_dkr"].shape == (80, 256)
    assert d["q"].shape == (2, 8, 48)
    assert list(d["q_positions"]) == [255, 255]
    assert d["slots"].tolist() == list(range(512))
    p = I.make(I.scaled(I.PREFILL, batch=2, seq_len=100, hidden=64, num_heads=4), 0)
    assert p["q"].shape == (200, 4, 192) and p["h"].dtype == np.uint16
    assert p["cu_seqlens"].tolist() == [0, 100, 200]
