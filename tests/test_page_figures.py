"""Cache-size closed forms against the figures the pages print (tests/golden/page_figures.json)."""
import json
import os

import pytest

from oracle import sizes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))
FIG = {f["id"]: f for f in GOLD["figures"]}
KiB, GiB, TiB = 1024.0, 1024.0 ** 3, 1024.0 ** 4


def _close(got, fig):
    tol = fig.get("tol", 0.0)
    assert abs(got - fig["value"]) <= tol * abs(fig["value"]) + 1e-12, (fig["id"], got, fig["value"])


def test_token_and_page_sizes():
    assert sizes.mla_elems_per_token(512, 64) == FIG["elems_per_token"]["value"]
    _close(sizes.mla_bytes_per_token(512, 64) / KiB, FIG["bytes_per_token"])
    _close(sizes.mha_bytes_per_token(128, 128) / KiB, FIG["mha_bytes_per_token"])
    _close(100 * sizes.compression(sizes.mla_bytes_per_token(512, 64),
                                   sizes.mha_bytes_per_token(128, 128)), FIG["compression_percent"])
    _close(sizes.page_bytes(16, 512, 64) / KiB, FIG["page16_bytes"])
    _close(sizes.page_bytes(64, 512, 64) / KiB, FIG["page64_bytes"])
    _close(sizes.staged_tile_bytes(64, 512, 64, 3) / KiB, FIG["three_stage_tile_bytes"])


def test_whole_model_cache_64k_b16():
    f = FIG["mha_cache_64k_b16"]
    _close(sizes.cache_bytes(sizes.mha_bytes_per_token(128, 128), 65536, 16, f["layers"]) / TiB, f)
    f = FIG["gqa8_cache_64k_b16"]
    _close(sizes.cache_bytes(sizes.gqa_bytes_per_token(8, 128), 65536, 16, f["layers"]) / GiB, f)
    f = FIG["mla_cache_64k_b16"]
    _close(sizes.cache_bytes(sizes.mla_bytes_per_token(512, 64), 65536, 16, f["layers"]) / GiB, f)


@pytest.mark.parametrize("seq_len", [4096, 16384, 65536])
def test_mha2mla_ratio(seq_len):
    f = FIG["mha2mla_ratio_percent"]
    mla = sizes.mla_bytes_per_token(64, 8) * seq_len
    mha = sizes.mha_bytes_per_token(32, 128) * seq_len
    _close(100 * mla / mha, f)


def test_workload_page_bytes_match_layout():
    import workloads as W
    for i, c in W.CONFIGS.items():
        per_tok = sizes.mla_bytes_per_token(c["d_c"], c["d_R"])
        assert per_tok == (1152 if c["d_c"] == 512 else 144)
        assert sizes.page_bytes(W.PAGE, c["d_c"], c["d_R"]) == (73728 if c["d_c"] == 512 else 9216)
