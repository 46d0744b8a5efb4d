"""Device-memory plumbing for paged KV caches: allocate the pool and summary
tensors with torch, upload host arrays, build page tables and the ABI
structs, and fill the cache through the library's own append entry point.

Nothing here computes any part of the method; it only moves bytes and calls
query_aware_sparse_amd's entry points.
"""
import numpy as np
import torch

from . import make_batch, make_cache, qas_append, qas_append_fp8

TORCH_KV = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "e4m3": torch.float8_e4m3fn}


def to_device(raw, dtype, device="cuda"):
    """Host raw storage array (see workloads) -> device tensor of `dtype`."""
    raw = np.ascontiguousarray(raw)
    if dtype == "bf16":
        t = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16)
    elif dtype == "e4m3":
        t = torch.from_numpy(raw.view(np.uint8)).view(torch.float8_e4m3fn)
    elif dtype == "f16":
        t = torch.from_numpy(raw.view(np.float16))
    else:
        t = torch.from_numpy(raw.astype(np.float32, copy=False))
    return t.to(device, non_blocking=False)


def ceil_div(a, b):
    return -(-int(a) // int(b))


class PagedCache:
    """A paged K/V pool with min/max summaries for one layer on the device.
    Unwritten slots are filled with NaN so that any read of a slot the
    method must not touch poisons the result."""

    def __init__(self, num_pool_pages, H_kv, S, d, kv_dtype, device="cuda",
                 poison=True, fp8_summaries=False):
        tdt = TORCH_KV[kv_dtype]
        shape = (num_pool_pages, H_kv, S, d)
        fill = float("nan") if poison else 0.0
        self.k_pool = torch.full(shape, fill, dtype=tdt, device=device)
        self.v_pool = torch.full(shape, fill, dtype=tdt, device=device)
        self.summary = torch.full((num_pool_pages, H_kv, 2, d), fill, dtype=tdt,
                                  device=device)
        self.summary_fp8 = self.summary_fp8_scale = None
        if fp8_summaries:   # e4m3 copy: codes 0x7F (NaN) and NaN scales until written
            self.summary_fp8 = torch.full((num_pool_pages, H_kv, 2, d), 0x7F, dtype=torch.uint8,
                                          device=device)
            self.summary_fp8_scale = torch.full((num_pool_pages, H_kv), fill, device=device)
        self.kv_dtype, self.S, self.H_kv, self.d = kv_dtype, S, H_kv, d
        self.device = device
        self.cache = make_cache(self.k_pool, self.v_pool, self.summary,
                                summary_fp8=self.summary_fp8,
                                summary_fp8_scale=self.summary_fp8_scale)


class DeviceBatch:
    """Page table and lengths of a batch on the device, with its qas_batch."""

    def __init__(self, lengths, pages, S, device="cuda"):
        lengths = np.asarray(lengths, dtype=np.int32)
        counts = [ceil_div(L, S) for L in lengths]
        indptr = np.zeros(len(lengths) + 1, dtype=np.int32)
        indptr[1:] = np.cumsum(counts)
        indices = np.concatenate([np.asarray(pages[r][:counts[r]], np.int32)
                                  for r in range(len(lengths))] + [np.zeros(0, np.int32)])
        self.lengths = lengths
        self.indptr_host = indptr
        self.seq_lens = torch.from_numpy(lengths).to(device)
        self.page_indptr = torch.from_numpy(indptr).to(device)
        self.page_indices = torch.from_numpy(
            indices if len(indices) else np.zeros(1, np.int32)).to(device)
        self.total_pages = int(indptr[-1])
        self.max_pages = int(max(counts)) if counts else 0
        self.batch = make_batch(self.seq_lens, self.page_indptr, self.page_indices,
                                self.total_pages, self.max_pages)


def prefill(pc, case, lengths=None, device="cuda"):
    """Write the first lengths[r] tokens of every request of a DecodeCase into
    the paged cache with qas_append (one call per request, so host memory
    stays bounded)."""
    lengths = case.seq_lens if lengths is None else np.asarray(lengths, np.int32)
    zeros = np.zeros(case.B, np.int32)
    before = DeviceBatch(zeros, case.pages, case.S, device)
    # the page table must cover the new tokens, lengths stay "before"
    full = DeviceBatch(lengths, case.pages, case.S, device)
    full_batch = make_batch(before.seq_lens, full.page_indptr, full.page_indices,
                            full.total_pages, full.max_pages)
    for r in range(case.B):
        n = int(lengths[r])
        if n == 0:
            continue
        new_indptr = np.zeros(case.B + 1, np.int32)
        new_indptr[r + 1:] = n
        k = to_device(case.keys[r][:n], case.kv_dtype, device)
        v = to_device(case.values[r][:n], case.kv_dtype, device)
        qas_append(pc.cache, full_batch, torch.from_numpy(new_indptr).to(device), n, n,
                   k, v)
        del k, v
    torch.cuda.synchronize()
    return full


def mfma_token_order(S):
    """Token at each k slot of a dim row of V^T, the B operand of the union
    kernel's PV MFMA: the slots a lane (row, hf) holds are (S/2) * hf + [0,
    S/2), and token t (w = t % 32, tau = t // 32) sits at slot (S/2) *
    ((w // 4) % 2) + 16 * tau + 4 * (w // 8) + w % 4."""
    order = np.empty(S, np.int64)
    for t in range(S):
        w, tau = t % 32, t // 32
        order[(S // 2) * ((w // 4) % 2) + 16 * tau + 4 * (w // 8) + w % 4] = t
    return order


def union_k_order(S, d=128):
    """Byte order of an fp8 K tile (one page, one KV head) for the union
    kernel: entry j of the stored tile is byte order[j] of the token-major
    [S][d] tile.  The tile is (S/32) * 2 * 2 blocks of 64 lanes x 16 bytes,
    block (tau, ks, c) giving lane (row = l % 32, hf = l // 32) bytes 16c +
    [0, 16) of its QK A operand: token 32 tau + row, dims 64 ks + 32 hf +
    16 c + [0, 16).  Each wave load is then 1 KiB of consecutive bytes."""
    assert d == 128 and S % 32 == 0
    order = np.empty(S * d, np.int64)
    j = 0
    for tau in range(S // 32):
        for ks in range(2):
            for c in range(2):
                for lane in range(64):
                    tok = 32 * tau + lane % 32
                    dim = 64 * ks + 32 * (lane // 32) + 16 * c
                    order[j:j + 16] = tok * d + dim + np.arange(16)
                    j += 16
    return order


def union_v_order(S, d=128):
    """Byte order of an fp8 V tile for the union kernel, from the
    token-major [S][d] tile: 4 * (S/32) blocks of 64 lanes x 16 bytes, block
    (dt, c) giving lane (row = l % 32, hf = l // 32) k slots (S/2) hf + 16 c
    + [0, 16) of dim row 32 dt + row of V^T (tokens in mfma_token_order)."""
    assert d == 128 and S % 32 == 0
    tok_at = mfma_token_order(S)
    order = np.empty(S * d, np.int64)
    j = 0
    for dt in range(4):
        for c in range(S // 32):
            for lane in range(64):
                dim = 32 * dt + lane % 32
                slots = (S // 2) * (lane // 32) + 16 * c + np.arange(16)
                order[j:j + 16] = tok_at[slots] * d + dim
                j += 16
    return order


class ChunkBatch:
    """Device state of one or more multi-query chunks (one per request) sharing
    an fp8 pool: pages of request r are placed after those of r - 1, each
    (page, KV head) tile of S * d bytes in the union kernel's operand order.

    writer="library" (default) quantises each request's float32 K/V with the
    per-head scales through qas_append_fp8, one call per request.
    writer="host" places the case's own e4m3 codes by plain copies in the
    order union_k_order / union_v_order give (no library call)."""

    def __init__(self, cases, device="cuda", writer="library"):
        c0 = cases[0]
        H, S, d = c0.H_kv, c0.S, c0.d
        self.S = S
        pool = sum(c.num_pool_pages for c in cases)
        shape = (pool, H, S, d)                     # sizes only: tiles are in operand order
        self.k_pool = torch.full(shape, 0x7F, dtype=torch.uint8, device=device)   # e4m3 NaN
        self.v_pool = torch.full(shape, 0x7F, dtype=torch.uint8, device=device)
        self.k_scale = torch.from_numpy(np.asarray(c0.k_scale, np.float32)).to(device)
        self.v_scale = torch.from_numpy(np.asarray(c0.v_scale, np.float32)).to(device)
        self.cache = make_cache(self.k_pool.view(torch.float8_e4m3fn),
                                self.v_pool.view(torch.float8_e4m3fn), None,
                                self.k_scale, self.v_scale)
        lengths, pages, off = [], [], 0
        for c in cases:
            P = ceil_div(c.L, S)
            lengths.append(c.L)
            pages.append(np.asarray(c.pages[:P], np.int32) + off)
            off += c.num_pool_pages
        if writer == "library":
            self._write_library(cases, lengths, pages, device)
        elif writer == "host":
            self._write_host(cases, lengths, pages, device)
        else:
            raise ValueError(f"unknown writer {writer!r}")
        self.db = DeviceBatch(lengths, pages, S, device)
        q_indptr = np.zeros(len(cases) + 1, np.int32)
        q_indptr[1:] = np.cumsum([c.N for c in cases])
        self.q_indptr = torch.from_numpy(q_indptr).to(device)
        self.q = to_device(np.concatenate([c.q for c in cases]), "bf16", device)
        self.q_pos = torch.from_numpy(np.concatenate([c.q_pos for c in cases])).to(device)
        self.sets = torch.from_numpy(np.ascontiguousarray(
            np.concatenate([c.sets for c in cases]), np.int32)).to(device)
        self.N = int(q_indptr[-1])
        self.group = c0.group

    def _write_library(self, cases, lengths, pages, device):
        B = len(cases)
        S = self.S
        before = DeviceBatch(np.zeros(B, np.int32), pages, S, device)
        full = DeviceBatch(lengths, pages, S, device)
        batch = make_batch(before.seq_lens, full.page_indptr, full.page_indices,
                           full.total_pages, full.max_pages)
        for r, c in enumerate(cases):
            if c.keys_src is None:
                raise ValueError("the library writer needs the case's float32 K/V")
            new_indptr = np.zeros(B + 1, np.int32)
            new_indptr[r + 1:] = c.L
            k = torch.from_numpy(np.ascontiguousarray(c.keys_src[:c.L], np.float32)).to(device)
            v = torch.from_numpy(np.ascontiguousarray(c.values_src[:c.L], np.float32)).to(device)
            qas_append_fp8(self.cache, batch, torch.from_numpy(new_indptr).to(device), c.L, c.L,
                           k, v)
            del k, v
        torch.cuda.synchronize()

    def _write_host(self, cases, lengths, pages, device):
        H, S, d = cases[0].H_kv, self.S, cases[0].d
        pool = self.k_pool.shape[0]
        korder = torch.from_numpy(union_k_order(S, d)).to(device)
        vorder = torch.from_numpy(union_v_order(S, d)).to(device)
        for c, pg in zip(cases, pages):
            P = len(pg)
            phys = torch.from_numpy(np.asarray(pg, np.int64)).to(device)
            for pool_t, raw, order in ((self.k_pool, c.keys, korder), (self.v_pool, c.values, vorder)):
                t = np.zeros((P * S, H, d), np.uint8)
                t[:c.L] = raw[:c.L]
                tt = torch.from_numpy(t).to(device).view(P, S, H, d).permute(0, 2, 1, 3)
                pool_t.view(pool, H, S * d)[phys] = tt.reshape(P, H, S * d)[..., order].contiguous()
