"""Seeded generators: determinism, per-sequence independence, shapes of the step's inputs."""
import numpy as np

from synth import configs, gen


def test_determinism_and_per_sequence_streams():
    cfg = configs.C1.scaled(B=3, T=16, n_comp=4, compress_rows=16)
    a = gen.queries(cfg)
    b = gen.queries(cfg)
    assert np.array_equal(a, b)
    one = gen.queries(cfg, seqs=[2])
    assert np.array_equal(one[0], a[2])
    assert not np.array_equal(a[0], a[1])


def test_compress_geometry_of_each_config():
    assert gen.compress_geometry(configs.C1) == (2048, 0, 0, 512)
    assert gen.compress_geometry(configs.C3) == (8, 1048576 - 8, 262143, 1)
    assert gen.compress_geometry(configs.C4) == (4100, 65532, 16384, 1024)
    assert gen.compress_geometry(configs.C4, hca=True) == (4096, 65536, 512, 32)
    assert gen.compress_geometry(configs.C5, hca=True) == (128, 1048576 - 128, 8191, 1)
    assert gen.compress_geometry(configs.C1, hca=True) == (2048, 0, 0, 16)


def test_storage_formats():
    cfg = configs.C3.scaled(n_comp=64, B=2)
    kc = gen.indexer_key_cache(cfg)
    assert kc["data"].dtype == np.uint8 and kc["data"].shape == (2, 64, 128)
    assert kc["scale"].dtype == np.float32 and kc["scale"].shape == (2, 64)
    cfg5 = configs.C5.scaled(n_comp=64, B=2)
    kc = gen.indexer_key_cache(cfg5)
    assert kc["data"].shape == (2, 64, 64) and kc["scale"].shape == (2, 64, 4)
    qi, w = gen.indexer_queries(cfg5)
    assert qi["data"].shape == (2, 1, 64, 64) and w.shape == (2, 1, 64)
    assert np.all((w >= 0) & (w < 1))
    assert gen.window(cfg).shape == (2, 128, 512) and gen.window(cfg).dtype == np.uint16
