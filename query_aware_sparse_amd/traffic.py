"""Algorithmic byte accounting of a decode-layer call (host arithmetic only).

Follows the Quest page's traffic model ("3.1.1 · Quest", §2, eq. (9)-(12)):
dense attention reads 2ML bytes, the summary scan 2MP (min and max per page,
i.e. 1/S of the keys), and the selected pages 2MKS, where M is the bytes of
one key or value vector.  To those the call's own I/O is added: the query and
output vectors and, when the current token is appended, the K/V row it
writes plus the tail page's summary it reads and rewrites.  Only the bytes
the method must move are counted; workspace traffic (scores, page lists,
split partials) is overhead and is not.
"""


def vector_bytes(d, elem_bytes):
    """M: bytes of one key or value vector of one head."""
    return d * elem_bytes


def dense_bytes(L, d, elem_bytes):
    """eq. (9): T_dense = 2 M L (one KV head)."""
    return 2 * vector_bytes(d, elem_bytes) * L


def summary_bytes(pages, d, elem_bytes):
    """eq. (10): T_index = 2 M P (one KV head)."""
    return 2 * vector_bytes(d, elem_bytes) * pages


def selected_bytes(selected_pages, S, d, elem_bytes):
    """eq. (11): T_selected = 2 M K S (one KV head)."""
    return 2 * vector_bytes(d, elem_bytes) * selected_pages * S


def read_ratio(S, K, P):
    """eq. (12): rho = 1/S + K/P."""
    return 1.0 / S + K / P


def fp8_summary_record_bytes(d):
    """One (page, KV head) record of the e4m3 summary copy ([Quest] §3,
    summary dtype): d min codes + d max codes + a 4-byte scale."""
    return 2 * d + 4


def decode_layer_bytes(*, B, H_q, H_kv, d, S, kv_bytes, q_bytes, pages_scanned,
                       page_heads_selected, append_tokens=0, fp8_summaries=False):
    """Bytes one decode-layer call moves by definition.

    pages_scanned: sum over requests of ceil(L_r / S) (summary records are
    read for every KV head).  page_heads_selected: sum over (request, KV head)
    of distinct valid selected pages.  append_tokens: tokens appended in the
    call (one per request for a decode step, or 0).  fp8_summaries: the scan
    reads the e4m3 copy instead of the exact records, and an append also
    writes the tail page's copy.  Returns a dict of parts and the total."""
    scan = (H_kv * pages_scanned * fp8_summary_record_bytes(d) if fp8_summaries
            else H_kv * summary_bytes(pages_scanned, d, kv_bytes))
    per_append = 2 * 2 * d * kv_bytes + 2 * 2 * d * kv_bytes
    if fp8_summaries:
        per_append += fp8_summary_record_bytes(d)
    parts = {
        "summary": scan,
        "selected_kv": selected_bytes(page_heads_selected, S, d, kv_bytes),
        "q_out": 2 * B * H_q * d * q_bytes,
        # K/V row read + written, tail summary record read + written (and
        # the tail's e4m3 copy written)
        "append": append_tokens * H_kv * per_append,
    }
    parts["total"] = sum(parts.values())
    return parts
