"""KV-cache size closed form.

Page "AI Data Engineering Pipeline, Part 8: Inference Optimization (vLLM)",
section "Phân Tích Cơ Cấu Bộ Nhớ Của KV Cache": one K and one V vector per KV
head, per layer, per token, each of head-dim elements; at 16-bit storage this
is 2*2*L*H_kv*d_k bytes per token. The Llama-3-70B shape (80 layers, 8 KV
heads, d_k 128) gives 327,680 bytes per token on that page.

Page "AI & MLOps Blog #54, LLM Inference Optimization", section 4's KV formula
multiplies by the byte width twice; this oracle follows the Part 8 form.
"""


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of K plus V for one token: 2 (K and V) * L * H_kv * d * bytes/elem."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def kv_bytes(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int, seq_len: int) -> int:
    """Memory_KV(S) for one sequence of S tokens."""
    return kv_bytes_per_token(num_layers, num_kv_heads, head_dim, elem_bytes) * seq_len
