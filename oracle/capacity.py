"""KV-cache byte accounting (oracle; test infrastructure only).

Citation keys are listed in ``oracle/__init__.py``.

Per-token cost ([SW] 知识点一; [LC] 1 "直觉与动机", 每 token 字节数;
[DQ] 07 "显存账本", the Cache_bytes formula): K and V each hold L layers x
H_kv heads x d values of s bytes, so c = 2 * L * H_kv * d * s bytes/token.

For B requests of lengths T_i ([SW] 知识点一, the three-ledger equations):
  useful = c * sum T_i
  padded = c * B * max T_i            (every request padded to the longest)
  paged  = c * b * sum ceil(T_i / b)  (independent b-token blocks)
and every non-empty request wastes fewer than b slots in its last block, so
the tail waste is below B (b - 1).  When physical blocks are shared, bytes
are counted over the set of unique physical blocks ([SW] 源码导读与边界推演).
"""


def _positive_int(name, x):
    if type(x) is not int or x < 1:
        raise ValueError(f"{name} must be a positive integer")


def bytes_per_token(layers, kv_heads, head_dim, element_bytes):
    """c = 2 * layers * kv_heads * head_dim * element_bytes (K and V)."""
    for name, x in (("layers", layers), ("kv_heads", kv_heads),
                    ("head_dim", head_dim), ("element_bytes", element_bytes)):
        _positive_int(name, x)
    return 2 * layers * kv_heads * head_dim * element_bytes


def paged_capacity(lengths, layers, kv_heads, head_dim, element_bytes, block_size):
    """Useful, padded and independently paged KV bytes for a set of requests.

    Lengths must be non-negative integers and all sizes positive integers
    (ValueError otherwise).  Returns a dict with keys: per_token, useful,
    padded, paged (bytes), slots (allocated token positions), blocks, and
    tail_waste (allocated minus useful positions).
    """
    lens = list(lengths)
    for n in lens:
        if type(n) is not int or n < 0:
            raise ValueError("lengths must be non-negative integers")
    _positive_int("block_size", block_size)
    c = bytes_per_token(layers, kv_heads, head_dim, element_bytes)
    useful_tokens = 0
    blocks = 0
    longest = 0
    for n in lens:
        useful_tokens += n
        blocks += -(-n // block_size)
        longest = max(longest, n)
    slots = blocks * block_size
    return {
        "per_token": c,
        "useful": c * useful_tokens,
        "padded": c * len(lens) * longest,
        "paged": c * slots,
        "slots": slots,
        "blocks": blocks,
        "tail_waste": slots - useful_tokens,
    }


def unique_block_bytes(block_tables, per_token, block_size):
    """Bytes of the distinct physical blocks referenced by the tables.

    ``block_tables`` is a list of per-request lists of physical block ids;
    a block referenced by several requests is counted once.
    """
    _positive_int("per_token", per_token)
    _positive_int("block_size", block_size)
    distinct = set()
    for row in block_tables:
        distinct.update(int(x) for x in row)
    return len(distinct) * block_size * per_token


def kv_cache_bytes(seq_len, layers, kv_heads, head_dim, element_bytes, batch):
    """Whole-batch cache: 2 * L * layers * H_kv * d * s * batch bytes."""
    _positive_int("batch", batch)
    if type(seq_len) is not int or seq_len < 0:
        raise ValueError("seq_len must be a non-negative integer")
    return seq_len * bytes_per_token(layers, kv_heads, head_dim, element_bytes) * batch


def mla_elements_per_token(d_c, d_rope):
    """Cached elements per token per layer for MLA: the latent plus the RoPE key."""
    _positive_int("d_c", d_c)
    _positive_int("d_rope", d_rope)
    return d_c + d_rope
