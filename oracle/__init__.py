"""CPU oracle for the TurboQuant hot path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct float64 NumPy implementation of what the GPU
path computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``oblivious_kv_cache_amd``) never imports, links or executes anything here,
and nothing here imports the product path: the two share no code, tables or
constant generators.  The only thing both sides consume is the seeded input
generator module ``oblivious_kv_cache_amd/workloads.py`` (random numbers and
byte patterns, none of the method's arithmetic), and that only through the
tests, which hand the same arrays to each side.

Sources (cited by page and section; the pages are Chinese-language web
articles about TurboQuant):
  * xujun.org note 189244, sections "第一步：PolarQuant" (random rotation,
    concentrated per-coordinate law), "第二步：QJL" (1-bit JL sketch of the
    residual, unbiased estimator with a full-precision query, 2/pi bias of the
    MSE-optimal 1-bit quantizer), "性能数据" (MSE within ~2.7x of the lower
    bound, ~1.45x at 1 bit), "常见问题" (data-oblivious; GloVe d=200 recall
    1@k).
  * suzuke blog "turboquant-compressing-ai-consciousness", section
    "技術上怎麼做到的": 第一步 (random orthogonal matrix, coordinates tend to
    N(0, 1/d)), 第二步 (Max-Lloyd codebook at b-1 bits), 第三步 (QJL sign
    projection of the residual; score = approximation + residual correction;
    3 bits -> MSE 0.03); "實際跑出來的數據" (online per-token compression).
  * hao.cnyes.com "TurboQuant", inline heading "1 bit 掃尾" (QJL keeps +1/-1
    per value and pairs it with an uncompressed query).

Functions whose result has no independent pin say "parity unpinned" in their
docstring.  Every other function is pinned by a ``-m "not gpu"`` test under
``tests/test_oracle_*.py``.
"""

from .rng import splitmix64_stream, gaussian_stream
from .params import (
    haar_rotation,
    jl_matrix,
    lloyd_max_gaussian,
    gaussian_distortion,
    codebook,
    TQParams,
    make_params,
)
from .quant import (
    record_sizes,
    pack_bits,
    unpack_bits,
    pack_planes,
    unpack_planes,
    pack_codes,
    unpack_codes,
    quantize_one,
    quantize,
    stage2_from_codes,
    dequant,
)
from .estimate import (
    prep_query,
    scores_one,
    scores,
    softmax,
    attend,
    topk,
    exact_top1,
    recall_at_k,
)

__all__ = [
    "splitmix64_stream", "gaussian_stream", "haar_rotation", "jl_matrix",
    "lloyd_max_gaussian", "gaussian_distortion", "codebook", "TQParams",
    "make_params", "record_sizes", "pack_bits", "unpack_bits", "pack_planes", "unpack_planes",
    "pack_codes", "unpack_codes", "quantize_one",
    "quantize", "stage2_from_codes", "dequant", "prep_query", "scores_one", "scores", "softmax",
    "attend", "topk", "exact_top1", "recall_at_k",
]
