"""KV-cache bytes per token, latent vs decompressed.

Test infrastructure only. mlxcel pull request 995, commit
"performance-validation report": the latent cache stores 8.89x fewer bytes
per token per layer than the decompressed per-head K/V, which moves the
longest context a 16 GiB KV budget holds from 62137 to 552336 tokens. The
geometry behind those numbers: latent width kv_lora_rank + qk_rope_head_dim
= 512 + 64 at 2 bytes; decompressed H * (qk_head_dim + v_head_dim) =
16 * (192 + 128) at 2 bytes (mlxcel pull request 995, the linked issue
text quoted after "Closes #907"); 27 layers.
"""


def latent_bytes_per_token(elem_bytes: int = 2, latent: int = 512, rope: int = 64) -> int:
    return (latent + rope) * elem_bytes


def decompressed_bytes_per_token(heads: int = 16, qk_head: int = 192, v_head: int = 128,
                                 elem_bytes: int = 2) -> int:
    return heads * (qk_head + v_head) * elem_bytes


def max_context_tokens(budget_bytes: int, bytes_per_token: int, layers: int) -> int:
    return budget_bytes // (bytes_per_token * layers)
