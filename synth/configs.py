"""Workload shapes for the CSA/HCA layer step.

Model sizes follow the DeepSeek-V4 hyper-parameter table in
"【论文解读】DeepSeek-V4" (wkq9411.github.io), section 三(二) "模型配置"
(Flash: 64 query heads, Pro: 128; head dim 512; indexer 64 heads x 128;
top-k 512 / 1024; m = 4, m' = 128; window 128), and the 1M-context entry
counts in "DeepseekV4论文解析" (blog.chaseai.de), section 2 "Hybrid Attention"
(262,144 CSA candidates, 1024+128 / 512+128 entries read, 8,192 HCA entries).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class CSAConfig:
    name: str
    B: int                 # sequences
    T: int                 # query rows per sequence (1 = decode)
    pos0: int              # absolute position of query row 0 (same for every sequence)
    n_comp: int            # compressed CSA entries in the cache (Nmax)
    c: int                 # head / KV dim
    H: int                 # query heads sharing one KV head
    HI: int                # indexer heads
    cI: int                # indexer head dim
    k: int                 # top-k
    rope_dims: int         # RoPE on the last rope_dims dims
    idx_dtype: str         # 'f32' | 'bf16' | 'fp8' | 'mxfp4'  (indexer q/k storage)
    kv_dtype: str          # 'f32' | 'bf16'                    (KV, q, outputs)
    m: int = 4             # CSA compression ratio
    n_win: int = 128       # sliding window
    m_hca: int = 128       # HCA compression ratio
    with_hca: bool = False  # step also runs one HCA layer
    n_hca: int = 0         # HCA entries in the cache
    compress_rows: int = 0  # per-token rows handed to csa_compress in the step (0 = none)
    rope_base: float = 10000.0
    eps: float = 1e-6
    seed: int = 0
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / (self.c ** 0.5)

    @property
    def decode(self) -> bool:
        return self.T == 1

    def visible(self, t: int) -> int:
        """Compressed CSA entries visible to absolute position t (s < floor(t/m))."""
        return min(t // self.m, self.n_comp)

    def scaled(self, **kw) -> "CSAConfig":
        return replace(self, **kw)


# C1: everything in fp32, small enough for the oracle to run every row.
C1 = CSAConfig(
    name="c1_tiny_prefill_fp32", B=1, T=2048, pos0=0, n_comp=512, c=128, H=8, HI=4, cI=32,
    k=64, rope_dims=32, idx_dtype="f32", kv_dtype="f32", compress_rows=2048,
    with_hca=True, m_hca=128, n_hca=16,
    description="tiny CSA prefill, fp32, n=2048, m=4, c=128, 8 heads, indexer 4x32, k=64, window 128, RoPE 32",
)

# C2: Flash-shaped decode at 128K context.
C2 = CSAConfig(
    name="c2_flash_decode_128k", B=32, T=1, pos0=131072, n_comp=32768, c=512, H=64, HI=64, cI=128,
    k=512, rope_dims=64, idx_dtype="bf16", kv_dtype="bf16", compress_rows=8,
    description="Flash decode, B=32, ctx 131072, 64 heads x 512, indexer 64x128 bf16, k=512",
)

# C3: Pro-shaped decode at 1M context, fp8 indexer with per-row scales.
C3 = CSAConfig(
    name="c3_pro_decode_1m_fp8", B=4, T=1, pos0=1048576, n_comp=262144, c=512, H=128, HI=64, cI=128,
    k=1024, rope_dims=64, idx_dtype="fp8", kv_dtype="bf16", compress_rows=8,
    description="Pro decode, B=4, ctx 1048576, 128 heads x 512, indexer 64x128 fp8 e4m3 + row scale, k=1024",
)

# C4: Flash-shaped chunked prefill: 65536 cached tokens + a 4096-token chunk, then HCA.
C4 = CSAConfig(
    name="c4_flash_chunked_prefill", B=1, T=4096, pos0=65536, n_comp=17408, c=512, H=64, HI=64, cI=128,
    k=512, rope_dims=64, idx_dtype="bf16", kv_dtype="bf16", compress_rows=4096 + 4,
    with_hca=True, m_hca=128, n_hca=544,
    description="Flash chunked prefill, 64K cached + 4K chunk, k=512 + SWA128, then HCA m'=128 over 544 entries",
)

# C5: Pro-shaped 1M decode with an MXFP4 indexer, CSA + HCA layers.
C5 = CSAConfig(
    name="c5_pro_decode_1m_mxfp4", B=8, T=1, pos0=1048576, n_comp=262144, c=512, H=128, HI=64, cI=128,
    k=1024, rope_dims=64, idx_dtype="mxfp4", kv_dtype="bf16", compress_rows=8,
    with_hca=True, m_hca=128, n_hca=8192,
    description="Pro decode 1M, B=8, MXFP4 indexer (e2m1 + E8M0 block-32), k=1024, CSA + HCA",
)

CONFIGS = {cfg.name: cfg for cfg in (C1, C2, C3, C4, C5)}
ALIASES = {"c1": C1.name, "c2": C2.name, "c3": C3.name, "c4": C4.name, "c5": C5.name}


def get_config(name: str) -> CSAConfig:
    return CONFIGS[ALIASES.get(name, name)]
