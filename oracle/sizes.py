"""Closed-form cache sizes of the layouts the pages compare (TEST INFRASTRUCTURE).

Each function is the plain definition of a storage size; the tests pin them to the
figures the pages print (``tests/golden/page_figures.json``).

  bhfrc.com/news/60867 S1: a token of one layer is stored as a 512-d latent plus a 64-d RoPE
    key (576 elements); multi-head attention stores K and V for 128 heads of width 128.
  bhfrc.com/news/60867 S3: a page holds 64 tokens (vs. 16).
  bhfrc.com/news/60867 S5: a pipeline stage holds a tile of [latent | RoPE] rows, and the
    on-chip budget is tile rows x row bytes x stages.
  lpnh.cn/news/2494972 S2.1, S4.2: MHA caches 2 n_h d_h elements per token, GQA 2 n_g d_h,
    MLA d_r + d_kv.
"""


def mla_elems_per_token(d_c, d_R):
    return d_c + d_R


def mla_bytes_per_token(d_c, d_R, elem_bytes=2):
    return (d_c + d_R) * elem_bytes


def mha_bytes_per_token(n_heads, d_head, elem_bytes=2):
    return 2 * n_heads * d_head * elem_bytes


def gqa_bytes_per_token(n_groups, d_head, elem_bytes=2):
    return 2 * n_groups * d_head * elem_bytes


def page_bytes(page_size, d_c, d_R, elem_bytes=2):
    return page_size * mla_bytes_per_token(d_c, d_R, elem_bytes)


def staged_tile_bytes(tile_rows, d_c, d_R, stages, elem_bytes=2):
    """On-chip bytes of a multi-stage pipeline of [latent | RoPE] tiles."""
    return (tile_rows * d_c + tile_rows * d_R) * elem_bytes * stages


def cache_bytes(bytes_per_token_layer, seq_len, batch, layers):
    """Whole-model cache: bytes per token per layer x tokens x sequences x layers."""
    return bytes_per_token_layer * seq_len * batch * layers


def compression(bytes_mla, bytes_mha):
    """Fraction of the MHA cache that MLA saves."""
    return 1.0 - bytes_mla / bytes_mha
