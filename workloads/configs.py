"""The workload shapes of the paged-KV attention path.

Shapes follow the pages' statement of the problem (nano-vllm's decode and
prefill calls, the 256-token block of its block manager, Qwen3-0.6B-like head
counts) and the length mixes given for each workload below.  The last one,
wide_gqa_decode, keeps qwen3_decode's sequences but groups 8 query heads per KV
head (Qwen3-32B's 64 / 8 / 128 attention), the case the decode kernel's MFMA
form is for.
"""

# name -> description of the sequence population and head geometry.
#   kind      "decode": every sequence gets one new token stored at position len-1
#             "prefill": every sequence has a cached prefix and n new tokens
#   lens      decode only: explicit list, ("uniform", lo, hi) or ("loguniform", lo, hi)
#   layers    number of transformer layers sharing one pool [2, layers, blocks, bs, H_kv, d]
CONFIGS = {
    "tiny_decode": dict(
        kind="decode", B=4, lens=[1, 7, 16, 33], block_size=16,
        H_q=4, H_kv=2, d=64, num_blocks=32, layers=1,
    ),
    "qwen3_decode": dict(
        kind="decode", B=256, lens=("uniform", 128, 2048), block_size=256,
        H_q=16, H_kv=8, d=128, layers=1,
    ),
    "long_decode": dict(
        kind="decode", B=32, lens=("uniform", 8192, 32768), block_size=256,
        H_q=16, H_kv=8, d=128, layers=1,
    ),
    "prefix_prefill": dict(
        kind="prefill", B=16, block_size=256, H_q=16, H_kv=8, d=128, layers=1,
        # cached prefix = 256 * U{0..16}; the first `shared_seqs` sequences take
        # 256 * U{8..16} and share their first `shared_blocks` physical blocks.
        prefix_blocks=(0, 16), shared_seqs=4, shared_blocks=8,
        new_tokens=(128, 2048),
    ),
    "full_step": dict(
        kind="decode", B=512, lens=("loguniform", 16, 16384), block_size=256,
        H_q=32, H_kv=8, d=128, layers=28,
    ),
    "wide_gqa_decode": dict(
        kind="decode", B=256, lens=("uniform", 128, 2048), block_size=256,
        H_q=64, H_kv=8, d=128, layers=1,
    ),
}

CONFIG_ORDER = ["tiny_decode", "qwen3_decode", "long_decode", "prefix_prefill", "full_step",
                "wide_gqa_decode"]


def config_seed(name: str) -> int:
    """Seed of a named workload: 1000 + its 1-based position in CONFIG_ORDER."""
    return 1000 + CONFIG_ORDER.index(name) + 1
