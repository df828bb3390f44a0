"""The five synthetic workloads of the Engram layer forward.

Every workload is seeded and synthetic. The shapes and the value distributions
follow what the pages state about the layer:

* vocabulary 129280 raw ids compressed to 99092 ids, n-gram orders 2..4 with
  8 heads each, the prime search base 16,000,000, 256-wide rows
  (page "Engram条件记忆：DeepSeek-V4.1-Flash中196B稀疏参数N-gram哈希查表的实现原理",
  the config.json table; page "DeepSeek-V4.1 模型结构（5）：记忆，Engram",
  section "一层只有一张表");
* 264-byte rows of 256 E4M3 bytes and 8 E8M0 block scales (page
  "ds4.c 学习笔记 · Engram", section "布局与哈希探测");
* 4 hyper-connection streams of width 5120 and the fused 6144 -> 5*5120
  projection (page "DeepSeek-V4.1 模型结构（5）：记忆，Engram", section
  "门控：用当前的上下文决定查到的向量用多少").

Token ids are finite Zipf(1.1) draws, standing in for natural-text token
streams, whose n-gram accesses one page calls Zipf-distributed (page
"DeepSeek Engram 详解：把静态知识从计算里拆出来", section 8.2). No tokenizer,
corpus or trained weight is used.

This module only describes shapes and seeds; it computes nothing of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

ROW_E4M3_E8M0 = "e4m3_e8m0_264"
ROW_F32 = "f32"


@dataclass(frozen=True)
class EngramWorkload:
    name: str
    description: str
    seed: int
    raw_vocab: int
    compressed_vocab: int
    max_ngram: int            # N: orders 2..N
    heads: int                # K heads per order
    prime_base: int           # primes are taken ascending from here (>= base)
    batch: int
    seq: int
    # DEAD layout: either fixed (start, end) spans applied to every sequence,
    # or (count, length) random non-overlapping spans per sequence.
    dead_fixed: Tuple[Tuple[int, int], ...] = ()
    dead_random: Tuple[int, int] = (0, 0)
    # seeds of the hash setup (token map + multipliers); None = own seed
    hash_setup_seed: Optional[int] = None
    # stages this workload exercises
    has_table: bool = False
    has_forward: bool = False
    row_format: str = ROW_E4M3_E8M0
    row_dim: int = 256
    hc: int = 4
    dim: int = 5120
    eps: float = 1e-6
    gate_clamp: float = 0.0
    zipf_s: float = 1.1
    decode_history: bool = False      # T = 1 tokens carrying a 3-token history
    dead_sequence0: bool = False      # decode: sequence 0 sits inside an image span
    table_seed: int = 0              # seed of the counter-based table generator
    extra: dict = field(default_factory=dict)

    @property
    def segments(self) -> int:
        return (self.max_ngram - 1) * self.heads

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def mem_dim(self) -> int:
        return self.segments * self.row_dim

    @property
    def kv_cols(self) -> int:
        return (self.hc + 1) * self.dim

    @property
    def setup_seed(self) -> int:
        return self.seed if self.hash_setup_seed is None else self.hash_setup_seed


C0 = EngramWorkload(
    name="C0",
    description="tiny CPU-checkable instance: V 128->97, orders 2-4 x 2 heads, "
                "primes from 1009, fp32 rows of 32, hc=1, width 64, 1x64 tokens",
    seed=1000, raw_vocab=128, compressed_vocab=97, max_ngram=4, heads=2,
    prime_base=1009, batch=1, seq=64, dead_fixed=((20, 28),),
    has_table=True, has_forward=True, row_format=ROW_F32, row_dim=32,
    hc=1, dim=64,
)

C1 = EngramWorkload(
    name="C1",
    description="hash/index only at full shape: V 129280->99092, 24 segments from "
                "16,000,000, 8x4096 Zipf tokens, 2 DEAD spans of 256 per sequence",
    seed=1001, raw_vocab=129280, compressed_vocab=99092, max_ngram=4, heads=8,
    prime_base=16_000_000, batch=8, seq=4096, dead_random=(2, 256),
)

C2 = EngramWorkload(
    name="C2",
    description="gather + dequant: 24 segments from 1,000,000 (24,003,916 rows x 264 B), "
                "16x8192 Zipf tokens, output bf16 [131072, 6144]",
    seed=1002, raw_vocab=129280, compressed_vocab=99092, max_ngram=4, heads=8,
    prime_base=1_000_000, batch=16, seq=8192, dead_random=(2, 256),
    hash_setup_seed=1001, has_table=True, table_seed=2002,
)

C3 = EngramWorkload(
    name="C3",
    description="full prefill layer forward: 4x8192 tokens, C2's table, wkv bf16 "
                "[6144 -> 5*5120], hc=4, width 5120",
    seed=1003, raw_vocab=129280, compressed_vocab=99092, max_ngram=4, heads=8,
    prime_base=1_000_000, batch=4, seq=8192, dead_random=(2, 256),
    hash_setup_seed=1001, has_table=True, has_forward=True, table_seed=2002,
)

C4 = EngramWorkload(
    name="C4",
    description="decode: 256 sequences x 1 token with a 3-token history against a "
                "full-size 384,006,168-row (101.4 GB) table, hc=4, width 5120",
    seed=1004, raw_vocab=129280, compressed_vocab=99092, max_ngram=4, heads=8,
    prime_base=16_000_000, batch=256, seq=1, hash_setup_seed=1001,
    has_table=True, has_forward=True, decode_history=True, dead_sequence0=True,
    table_seed=2004,
)

WORKLOADS = {w.name: w for w in (C0, C1, C2, C3, C4)}
