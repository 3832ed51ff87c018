"""The seeded input generator: determinism, valid page tables, poison placement."""
import numpy as np
import torch

import workloads as W


def test_deterministic():
    a = W.make_inputs(3, 4, 8, 16, 4, 8, ("uniform", 5, 200), 7)
    b = W.make_inputs(3, 4, 8, 16, 4, 8, ("uniform", 5, 200), 7)
    for k in ("q_nope", "q_rope", "W_UK", "W_UV", "kv_pages", "page_table", "seq_lens"):
        assert torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k],
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k])


def test_page_table_is_injective_into_pool():
    inp = W.make_inputs(5, 2, 4, 8, 2, 4, [1, 64, 65, 200, 3], 3, poison=True)
    used = []
    for b in range(5):
        n = -(-int(inp["seq_lens"][b]) // 64)
        used += inp["page_table"][b, :n].tolist()
    assert len(set(used)) == len(used) == inp["used_pages"]
    assert all(0 <= p < inp["pool_pages"] for p in inp["page_table"].flatten().tolist())
    assert inp["pool_pages"] > inp["used_pages"]


def test_poison_only_outside_sequences():
    inp = W.make_inputs(3, 2, 4, 8, 2, 4, [1, 70, 128], 4, poison=True)
    kv = inp["kv_pages"].float()
    P = inp["page_size"]
    for b in range(3):
        S = int(inp["seq_lens"][b])
        for t in range(-(-S // P) * P):
            pg = int(inp["page_table"][b, t // P])
            assert bool(torch.isnan(kv[pg, t % P]).all()) == (t >= S)
    # spare pages are entirely NaN
    live = set()
    for b in range(3):
        live |= set(inp["page_table"][b, :-(-int(inp["seq_lens"][b]) // P)].tolist())
    for p in range(inp["pool_pages"]):
        if p not in live:
            assert torch.isnan(kv[p]).all()


def test_distributions():
    inp = W.make_inputs(2, 128, 128, 512, 64, 128, [512, 512], 0)
    assert abs(inp["W_UK"].float().std().item() - 512 ** -0.5) < 1e-3
    assert abs(inp["q_nope"].float().std().item() - 1.0) < 2e-2
    assert abs(inp["kv_pages"].float().std().item() - 1.0) < 1e-2


def test_config_shapes():
    c = W.CONFIGS
    assert (c[2]["B"], c[2]["seq"]) == (16, ("fixed", 4096))
    assert c[5]["d_c"] + c[5]["d_R"] == 72 and c[5]["d_n"] + c[5]["d_R"] == 128
    inp = W.config_inputs(1)
    assert inp["page_table"].tolist() == [list(range(8))]
    assert inp["kv_pages"].shape == (8, 64, 576)
