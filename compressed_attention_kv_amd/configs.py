"""The workloads the hot path is checked and measured on.

Shapes follow the DeepSeek-V4 attention block as the V4-Pro architecture card
(llm-arch-kb, "What's new in V4", §1 Hybrid attention) gives it: 128 query
heads of dim 512 sharing one KV head, CSA compression m=4 with a 64-head
dim-128 Lightning Indexer keeping k=1024 entries, HCA compression m'=128, a
128-token raw window, per-head sinks, and rotary embedding on the last 64
dims.  Context lengths (128K, 1M) and batch sizes are synthetic stand-ins for
the long-context runs the pages discuss.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int                 # sequences
    Q: int                 # query tokens per sequence
    H: int = 128           # query heads
    D: int = 512           # head dim (shared KV head dim)
    rope_dims: int = 64
    rope_base: float = 10000.0
    n_win: int = 128
    m: int = 4             # CSA compression ratio
    m_hca: int = 128       # HCA compression ratio
    HI: int = 64           # indexer heads
    dI: int = 128          # indexer head dim
    k: int = 1024          # top-k
    dtype: str = "bf16"    # activation storage type: "bf16" or "f32"
    csa: bool = True
    hca: bool = False
    prefill: bool = False
    T: int = 0             # prefill: raw tokens per sequence (prefix + chunk)
    q_pos0: int = 0        # prefill: position of the first query
    N: int = 0             # decode: compressed entries per sequence
    t: int = 0             # decode: query position (context length)
    fp8_index: bool = True # indexer keys stored as fp8 E4M3 + per-entry scale
    rms_eps: float = 1e-6

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def decode(self) -> bool:
        return not self.prefill


WORKLOADS = {
    # tiny CSA layer in fp32: 2048-token causal prefill, m=4 -> 512 entries
    "tiny_csa_f32": Workload(
        name="tiny_csa_f32", seed=0, B=1, Q=2048, H=8, D=128, rope_dims=32, n_win=16,
        HI=4, dI=32, k=64, dtype="f32", prefill=True, T=2048, q_pos0=0, fp8_index=False),
    # CSA decode at 128K context: 32 sequences, 32768 compressed entries each
    "csa_decode_128k": Workload(
        name="csa_decode_128k", seed=1, B=32, Q=1, N=32768, t=131072),
    # HCA decode at 1M context: 32 sequences, 8192 compressed entries each
    "hca_decode_1m": Workload(
        name="hca_decode_1m", seed=2, B=32, Q=1, N=8192, t=1048576, m=128, csa=False, hca=True),
    # CSA decode at 1M context: 8 sequences, 262144 compressed entries each
    "csa_decode_1m": Workload(
        name="csa_decode_1m", seed=3, B=8, Q=1, N=262144, t=1048576),
    # CSA + HCA chunked prefill: 8192 new tokens after a 262144-token prefix
    "prefill_chunk_256k": Workload(
        name="prefill_chunk_256k", seed=4, B=1, Q=8192, prefill=True, T=262144 + 8192,
        q_pos0=262144, csa=True, hca=True),
    # V4-Flash attention shapes ("DeepSeek V4-Pro" card, Family: 64 query
    # heads, CSA top-k 512) at the same contexts as the V4-Pro decode workloads
    "flash_csa_decode_128k": Workload(
        name="flash_csa_decode_128k", seed=5, B=32, Q=1, N=32768, t=131072, H=64, k=512),
    "flash_hca_decode_1m": Workload(
        name="flash_hca_decode_1m", seed=6, B=32, Q=1, N=8192, t=1048576, m=128, csa=False, hca=True, H=64),
}


def get_workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.replace(**overrides) if overrides else w
