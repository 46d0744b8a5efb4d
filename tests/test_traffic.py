"""Byte accounting against the Quest page's own traffic example (§2)."""
from query_aware_sparse_amd import traffic
from tests.conftest import load_golden


def test_pages_traffic_example():
    g = load_golden("quest_traffic.json")
    L, S, K, d, e = g["L"], g["S"], g["K"], g["d"], g["bytes_per_elem"]
    P = L // S
    MiB = 1 << 20
    assert traffic.vector_bytes(d, e) == g["vector_bytes"]
    assert traffic.dense_bytes(L, d, e) == g["dense_MiB"] * MiB
    assert traffic.summary_bytes(P, d, e) == g["summary_MiB"] * MiB
    assert traffic.selected_bytes(K, S, d, e) == g["selected_MiB"] * MiB
    assert traffic.read_ratio(S, K, P) == g["rho"]
    rho = (traffic.summary_bytes(P, d, e) + traffic.selected_bytes(K, S, d, e)) \
        / traffic.dense_bytes(L, d, e)
    assert rho == g["rho"]


def test_llama_layer_call_bytes():
    """The 32K-context, K=256, 32x128-head fp16 layer call: 32 MiB of
    summaries, 64 MiB of selected K/V and 16 KiB of q/o."""
    p = traffic.decode_layer_bytes(B=1, H_q=32, H_kv=32, d=128, S=16, kv_bytes=2,
                                   q_bytes=2, pages_scanned=2048,
                                   page_heads_selected=32 * 256)
    assert p["summary"] == 33554432 and p["selected_kv"] == 67108864
    assert p["q_out"] == 16384 and p["total"] == 100679680
