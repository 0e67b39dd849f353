"""The five workloads: shapes and hyper-parameters in the pages' notation.

Hyper-parameters B=64, l_C1=B/2, s_C1=B/4, l=5, s=4 follow the three-stage
compression of the papernotes.org InfLLM-V2 note (方法详解 > 关键设计 3);
N_init, N_local and k follow its key design 2.  Shapes h_q=32, h_kv=2, d=128
follow the 8B GQA backbone in the same note (实验关键数据).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    n_q: int            # query tokens per sequence
    n_kv: int           # keys per sequence (cache length for decode)
    h_q: int
    h_kv: int
    d: int
    io: str             # "bf16" | "f32"
    k: int
    n_needles: int      # planted needle blocks per sequence
    seed: int
    B: int = 64
    l_C1: int = 32
    s_C1: int = 16
    l: int = 5
    s: int = 4
    N_init: int = 1
    N_local: int = 2
    decode: bool = False
    notes: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.h_q // self.h_kv

    @property
    def q_pos0(self) -> int:
        """Absolute position of query token 0 (decode: the new token L-1)."""
        return self.n_kv - self.n_q

    @property
    def n_blk(self) -> int:
        return -(-self.n_kv // self.B)


CONFIGS = {
    "tiny": Config("tiny", batch=1, n_q=2048, n_kv=2048, h_q=8, h_kv=2, d=64, io="f32",
                   k=4, n_needles=4, seed=1001,
                   notes="tiny causal prefill, fp32, G=4"),
    "prefill32k": Config("prefill32k", batch=1, n_q=32768, n_kv=32768, h_q=32, h_kv=2, d=128,
                         io="bf16", k=16, n_needles=32, seed=1002,
                         notes="MiniCPM-style GQA layer prefill at 32k"),
    "prefill128k": Config("prefill128k", batch=1, n_q=131072, n_kv=131072, h_q=32, h_kv=2,
                          d=128, io="bf16", k=16, n_needles=64, seed=1003,
                          notes="long prefill at 128k"),
    "decode": Config("decode", batch=16, n_q=1, n_kv=131072, h_q=32, h_kv=2, d=128, io="bf16",
                     k=16, n_needles=16, seed=1004, decode=True,
                     notes="decode step, 16 sequences, 128k cache each"),
    "dense_switch": Config("dense_switch", batch=8, n_q=4096, n_kv=4096, h_q=32, h_kv=2, d=128,
                           io="bf16", k=64, n_needles=0, seed=1005,
                           notes="short sequences: init+local+top-k covers every block"),
}
