"""The five synthetic DSA workloads (shapes, value distributions, structure).

Each workload follows the DeepSeek Sparse Attention problem statement: a
lightning indexer scores every causally visible key with H_I FP8 heads
(DeepSeek-V3.2-Exp summary page, section "Method"), the top-k = 2048 keys per
query are kept (AMD MI355X article, section "Fine-Grained Token Selection";
same summary page, "Method"), and MLA in MQA mode attends over only those
latent KV rows.  Shapes, distributions and the paging block size are the
workload definitions of this project; the pages give none of them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" (one sequence, T queries) or "decode"
    T: int                    # query tokens (decode: number of sequences)
    S: int                    # keys in context (decode: max context length)
    q_start: int              # absolute position of query row 0 (prefill)
    H_I: int                  # indexer heads
    D_I: int                  # indexer head dim
    topk: int
    H: int                    # MLA query heads
    D_qk: int                 # latent + rope width of one KV row
    D_v: int                  # value width (leading columns of the same row)
    sm_scale: float
    outlier_frac: float = 0.0     # fraction of indexer-key rows scaled before quantization
    outlier_factor: float = 1.0
    decode_len_lo: int = 0        # decode: context lengths drawn in [lo, hi]
    decode_len_hi: int = 0
    block_size: int = 64          # paged-cache block size
    seed: int = 0
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload(
        name="tiny", kind="prefill", T=256, S=256, q_start=0, H_I=4, D_I=32, topk=64,
        H=8, D_qk=80, D_v=64, sm_scale=1.0 / math.sqrt(80.0),
        notes="L=256 causal correctness case; latent 64 + rope 16"),
    "prefill_4k": Workload(
        name="prefill_4k", kind="prefill", T=4096, S=4096, q_start=0, H_I=64, D_I=128,
        topk=2048, H=128, D_qk=576, D_v=512, sm_scale=1.0 / math.sqrt(192.0),
        notes="L=4096 causal; rows t < 2048 select every visible key"),
    "prefill_32k": Workload(
        name="prefill_32k", kind="prefill", T=32768, S=32768, q_start=0, H_I=64, D_I=128,
        topk=2048, H=128, D_qk=576, D_v=512, sm_scale=1.0 / math.sqrt(192.0),
        notes="L=32768 causal prefill, batch 1"),
    "decode_64": Workload(
        name="decode_64", kind="decode", T=64, S=131072, q_start=0, H_I=64, D_I=128,
        topk=2048, H=128, D_qk=576, D_v=512, sm_scale=1.0 / math.sqrt(192.0),
        decode_len_lo=8192, decode_len_hi=131072,
        notes="64 sequences x 1 new token, paged cache of 64-token blocks"),
    "chunked_131k": Workload(
        name="chunked_131k", kind="prefill", T=8192, S=131072, q_start=122880, H_I=64,
        D_I=128, topk=2048, H=128, D_qk=576, D_v=512, sm_scale=1.0 / math.sqrt(192.0),
        outlier_frac=0.01, outlier_factor=8.0,
        notes="8192 new queries at positions 122880..131071; 1% of key rows x8"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def visible(w: Workload, t: int) -> int:
    """Number of keys query row t sees: itself and every earlier position."""
    return min(w.S, w.q_start + t + 1)
