"""Seeded synthetic inputs (numpy PCG64, one SeedSequence child per tensor and sequence).

Recipe (shapes from ``synth.configs``):

* per-token compression streams C^a, C^b, Z^a, Z^b (KV dim c) and the indexer
  streams (dim c^I): N(0, 1); positional biases B^a, B^b (and HCA's B): N(0, 1);
* compressed KV cache and indexer-key cache entries not produced inside the
  step: N(0, 1);
* attention queries q ~ N(0, 1) / sqrt(c); indexer queries q^I ~ N(0, 1) / sqrt(c^I);
* indexer head weights w ~ U(0, 1); sink logits z' ~ N(0, 1); RMSNorm gains = 1
  (passed as NULL);
* window KV: N(0, 1), one row per position pos0-n_win+1 .. pos0+T-1.

Values are drawn in float32 and then stored in the workload's format: float32,
bf16 (round to nearest even), fp8 e4m3 with a per-row scale, or MXFP4 (both
quantized from the bf16-rounded Gaussians).  Every array is generated per
sequence from its own child seed, so any one sequence can be regenerated alone.
"""
from __future__ import annotations

import numpy as np

from . import formats
from .configs import CSAConfig

STREAMS = (
    "ca", "cb", "za", "zb", "bias_a", "bias_b",
    "ica", "icb", "iza", "izb", "ibias_a", "ibias_b",
    "kv_cache", "ik_cache", "q", "qi", "w", "win", "sink",
    "hca_c", "hca_z", "hca_bias", "hca_cache", "hca_q", "hca_win", "hca_sink",
    "extra0", "extra1", "extra2", "extra3",
    "dq", "dqi", "dw", "dhq",
    "cq", "w_uq", "w_iuq", "att_o", "w_g", "w_o",
)
_SID = {name: i for i, name in enumerate(STREAMS)}


def rng(seed: int, stream: str, b: int = 0) -> np.random.Generator:
    """Generator for tensor `stream`, sequence `b` (independent of every other pair)."""
    child = np.random.SeedSequence(seed).spawn(len(STREAMS))[_SID[stream]]
    return np.random.Generator(np.random.PCG64(child.spawn(b + 1)[b]))


def normal(seed, stream, shape, b=0, scale=1.0) -> np.ndarray:
    x = rng(seed, stream, b).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def uniform(seed, stream, shape, b=0) -> np.ndarray:
    return rng(seed, stream, b).random(size=shape, dtype=np.float32)


def store(x: np.ndarray, dtype: str):
    """float32 -> storage format.  Returns a dict of arrays (``data`` and, if any, ``scale``)."""
    if dtype == "f32":
        return {"data": np.ascontiguousarray(x, dtype=np.float32)}
    bits = formats.f32_to_bf16_bits(x)
    if dtype == "bf16":
        return {"data": bits}
    xb = formats.bf16_bits_to_f32(bits)
    if dtype == "fp8":
        codes, scale = formats.fp8_rowscale_encode(xb)
        return {"data": codes, "scale": scale}
    if dtype == "mxfp4":
        packed, sc = formats.mxfp4_encode(xb)
        return {"data": packed, "scale": sc}
    raise ValueError(dtype)


def per_seq(cfg: CSAConfig, stream: str, shape, dtype: str, scale: float = 1.0, dist: str = "normal",
            seqs=None):
    """Stack per-sequence draws of `shape` into [len(seqs), *shape] in storage format."""
    seqs = range(cfg.B) if seqs is None else seqs
    parts = []
    for b in seqs:
        if dist == "normal":
            x = normal(cfg.seed, stream, shape, b=b, scale=scale)
        else:
            x = uniform(cfg.seed, stream, shape, b=b)
        parts.append(store(x, dtype))
    return {key: np.stack([p[key] for p in parts]) for key in parts[0]}


def compress_geometry(cfg: CSAConfig, hca: bool = False):
    """(rows, row0_pos, first_entry, num_entries) of the csa_compress call inside the step."""
    if hca:
        mm = cfg.m_hca
        if cfg.T == 1:            # decode: the block that ends at pos0-1 completes now
            return mm, cfg.pos0 - mm, cfg.pos0 // mm - 1, 1
        if cfg.pos0 == 0:         # whole-sequence prefill
            return cfg.T, 0, 0, cfg.T // mm
        return cfg.T, cfg.pos0, cfg.pos0 // mm, cfg.T // mm
    m = cfg.m
    if cfg.T == 1:
        return 2 * m, cfg.pos0 - 2 * m, cfg.pos0 // m - 1, 1
    if cfg.pos0 == 0:
        return cfg.T, 0, 0, cfg.T // m
    # chunk plus the previous block's rows (needed for the b-stream of the first new entry)
    return cfg.T + m, cfg.pos0 - m, cfg.pos0 // m, cfg.T // m


def compress_inputs(cfg: CSAConfig, indexer: bool = False, hca: bool = False, seqs=None):
    """Per-token streams and biases for the step's csa_compress call, in cfg.kv_dtype."""
    dt = cfg.kv_dtype
    rows, row0, first, num = compress_geometry(cfg, hca)
    if hca:
        c = cfg.c
        out = {
            "ca": per_seq(cfg, "hca_c", (rows, c), dt, seqs=seqs)["data"],
            "za": per_seq(cfg, "hca_z", (rows, c), dt, seqs=seqs)["data"],
            "cb": None, "zb": None,
            "bias_a": normal(cfg.seed, "hca_bias", (cfg.m_hca, c)),
            "bias_b": None, "m": cfg.m_hca,
        }
    else:
        c = cfg.cI if indexer else cfg.c
        p = "i" if indexer else ""
        out = {
            "ca": per_seq(cfg, p + "ca", (rows, c), dt, seqs=seqs)["data"],
            "cb": per_seq(cfg, p + "cb", (rows, c), dt, seqs=seqs)["data"],
            "za": per_seq(cfg, p + "za", (rows, c), dt, seqs=seqs)["data"],
            "zb": per_seq(cfg, p + "zb", (rows, c), dt, seqs=seqs)["data"],
            "bias_a": normal(cfg.seed, p + "bias_a", (cfg.m, c)),
            "bias_b": normal(cfg.seed, p + "bias_b", (cfg.m, c)),
            "m": cfg.m,
        }
    out.update(rows=rows, row0_pos=row0, first_entry=first, num_entries=num, c=c, dtype=dt)
    return out


def kv_cache(cfg: CSAConfig, seqs=None, hca: bool = False):
    n = cfg.n_hca if hca else cfg.n_comp
    return per_seq(cfg, "hca_cache" if hca else "kv_cache", (n, cfg.c), cfg.kv_dtype, seqs=seqs)["data"]


def indexer_key_cache(cfg: CSAConfig, seqs=None):
    """K^IComp [B][N][c^I] in cfg.idx_dtype; dict with data (+ scale)."""
    return per_seq(cfg, "ik_cache", (cfg.n_comp, cfg.cI), cfg.idx_dtype, seqs=seqs)


def indexer_queries(cfg: CSAConfig, seqs=None):
    """q^I [B][T][HI][c^I] in cfg.idx_dtype (scale per (t, h) row for fp8), w [B][T][HI] fp32."""
    qi = per_seq(cfg, "qi", (cfg.T, cfg.HI, cfg.cI), cfg.idx_dtype, scale=1.0 / np.sqrt(cfg.cI), seqs=seqs)
    w = per_seq(cfg, "w", (cfg.T, cfg.HI), "f32", dist="uniform", seqs=seqs)["data"]
    return qi, w


def queries(cfg: CSAConfig, seqs=None, hca: bool = False):
    return per_seq(cfg, "hca_q" if hca else "q", (cfg.T, cfg.H, cfg.c), cfg.kv_dtype,
                   scale=1.0 / np.sqrt(cfg.c), seqs=seqs)["data"]


def window(cfg: CSAConfig, seqs=None, hca: bool = False):
    """Window KV [B][T+n_win-1][c]; row j holds position pos0 - n_win + 1 + j."""
    return per_seq(cfg, "hca_win" if hca else "win", (cfg.T + cfg.n_win - 1, cfg.c), cfg.kv_dtype,
                   seqs=seqs)["data"]


def sink(cfg: CSAConfig, hca: bool = False) -> np.ndarray:
    return normal(cfg.seed, "hca_sink" if hca else "sink", (cfg.H,))


def positions(cfg: CSAConfig) -> np.ndarray:
    return np.full((cfg.B,), cfg.pos0, dtype=np.int64)


def decode_streams(cfg: CSAConfig, length: int, b: int):
    """Every per-token row of sequence b for positions [0, length), as a decode loop consumes them (bf16 bits):
    the CSA KV streams ca, cb, za, zb [L][c], the indexer streams ica .. izb [L][cI], the HCA streams hca_c,
    hca_z [L][c], and the window KV rows of the CSA and HCA layers, win and hca_win [L][c].  N(0, 1)."""
    out = {}
    for name, width in (("ca", cfg.c), ("cb", cfg.c), ("za", cfg.c), ("zb", cfg.c), ("ica", cfg.cI), ("icb", cfg.cI),
                        ("iza", cfg.cI), ("izb", cfg.cI), ("hca_c", cfg.c), ("hca_z", cfg.c), ("win", cfg.c),
                        ("hca_win", cfg.c)):
        out[name] = store(normal(cfg.seed, name, (length, width), b=b), "bf16")["data"]
    return out


def decode_biases(cfg: CSAConfig):
    """The positional biases B^a, B^b (KV and indexer) and HCA's B, float32 [m][width]."""
    return {"bias_a": normal(cfg.seed, "bias_a", (cfg.m, cfg.c)), "bias_b": normal(cfg.seed, "bias_b", (cfg.m, cfg.c)),
            "ibias_a": normal(cfg.seed, "ibias_a", (cfg.m, cfg.cI)),
            "ibias_b": normal(cfg.seed, "ibias_b", (cfg.m, cfg.cI)),
            "hca_bias": normal(cfg.seed, "hca_bias", (cfg.m_hca, cfg.c))}


def decode_queries(cfg: CSAConfig, steps: int, b: int):
    """Per-step query rows of sequence b: q and hca q [S][H][c] (N(0,1)/sqrt(c)), indexer queries [S][HI][cI]
    (N(0,1)/sqrt(cI)) in the workload's indexer format, weights [S][HI] U(0, 1)."""
    q = store(normal(cfg.seed, "dq", (steps, cfg.H, cfg.c), b=b, scale=1.0 / np.sqrt(cfg.c)), "bf16")["data"]
    hq = store(normal(cfg.seed, "dhq", (steps, cfg.H, cfg.c), b=b, scale=1.0 / np.sqrt(cfg.c)), "bf16")["data"]
    qi = store(normal(cfg.seed, "dqi", (steps, cfg.HI, cfg.cI), b=b, scale=1.0 / np.sqrt(cfg.cI)), cfg.idx_dtype)
    w = uniform(cfg.seed, "dw", (steps, cfg.HI), b=b)
    return {"q": q, "hq": hq, "qi": qi, "w": w}


def proj_inputs(rows: int, d_c: int, n_h: int, c: int, n_hI: int, cI: int, g: int, d_g: int, d: int, seed: int = 0):
    """Synthetic inputs of the projections, bf16 bits: the latent c^Q [rows][d_c] and attention outputs
    [rows][n_h * c] ~ N(0, 1); output-major weights W^UQ [n_h c][d_c], W^IUQ [n_hI cI][d_c], the group
    projections [g][d_g][n_h c / g] and the final one [d][g d_g], each ~ N(0, 1) / sqrt(fan-in), so that
    every output is O(1)."""
    w = lambda name, shape, fan_in: store(normal(seed, name, shape, scale=1.0 / np.sqrt(fan_in)), "bf16")["data"]
    return {"cq": store(normal(seed, "cq", (rows, d_c)), "bf16")["data"],
            "w_uq": w("w_uq", (n_h * c, d_c), d_c), "w_iuq": w("w_iuq", (n_hI * cI, d_c), d_c),
            "o": store(normal(seed, "att_o", (rows, n_h * c)), "bf16")["data"],
            "w_g": w("w_g", (g, d_g, n_h * c // g), n_h * c // g), "w_o": w("w_o", (d, g * d_g), g * d_g)}
