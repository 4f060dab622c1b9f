"""The seeded input generators: determinism, shapes, ignore counts, document packing."""
import numpy as np
import torch

from reduction_rmsnorm_fwd_amd import synth


def test_deterministic_and_independent_streams():
    a = synth.normal_f32(7, 1, 1000)
    b = synth.normal_f32(7, 1, 1000)
    c = synth.normal_f32(7, 2, 1000)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # a prefix is the same draw whatever the total length (block streams)
    big = synth.normal_f32(7, 1, synth.BLOCK + 5)
    assert np.array_equal(big[:1000], a)


def test_moments():
    x = synth.normal_f32(0, 11, 1 << 20, std=3.0)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 3.0) < 0.02
    w = synth.normal_f32(0, 3, 1 << 16, std=0.1, mean=1.0)
    assert abs(w.mean() - 1.0) < 0.002 and abs(w.std() - 0.1) < 0.002


def test_ignore_counts_exact():
    for cid, n_ign in [(1, 0), (4, 4096), (5, 819)]:
        t = synth.targets(synth.CONFIGS[cid])
        assert int((t == synth.IGNORE_INDEX).sum()) == n_ign
        v = t[t != synth.IGNORE_INDEX]
        assert int(v.min()) >= 0 and int(v.max()) < synth.CONFIGS[cid].V


def test_packed_positions():
    cfg = synth.CONFIGS[4]
    lens = synth.doc_lengths_geometric(cfg.seed, cfg.T)
    assert sum(lens) == cfg.T and max(lens) <= 16384
    pos = synth.positions(cfg).numpy()
    starts = np.nonzero(pos == 0)[0]
    assert len(starts) == len(lens) and starts[0] == 0
    assert np.all(np.diff(pos)[np.diff(pos) != 1] <= 0)  # only resets break the ramp
    # mean document length in a long draw is ~1024
    many = synth.doc_lengths_geometric(99, 2_000_000)
    assert 950 < np.mean(many[:-1]) < 1100


def test_unpacked_positions_restart_per_document():
    pos = synth.positions(synth.CONFIGS[2]).numpy()
    assert np.array_equal(pos, np.concatenate([np.arange(2048), np.arange(2048)]))


def test_dtypes_and_shapes():
    cfg = synth.scaled(synth.CONFIGS[3], 16)
    x = synth.rmsnorm_inputs(cfg)
    assert x["x"].dtype == torch.bfloat16 and x["x"].shape == (16, 4096)
    r = synth.rope_inputs(cfg)
    assert r["q"].shape == (16, 32, 128) and r["k"].shape == (16, 8, 128)
    c1 = synth.rmsnorm_inputs(synth.CONFIGS[1])
    assert c1["x"].dtype == torch.float32
