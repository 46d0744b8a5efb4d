"""GPU parity of the FP8 E4M3 writer of the multi-query chunk path
(qas_append_fp8, PageWeaver notes SS2UKVF2: FP8 E4M3 K/V with a per-KV-head
scale): the codes it writes equal the oracle's quantisation code for code,
in the tile order qas.h documents for qas_chunk_attention, through bulk and
single-token appends that open, extend and cross pages; a cache it builds
equals, byte for byte, one placed from the workload's own codes; and the
chunk call reads it correctly (the other chunk tests run on such caches)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import quest
from tests.gpu_util import say
from workloads import multiquery_chunk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qas():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import query_aware_sparse_amd
    return query_aware_sparse_amd


# Tile layout as qas.h states it for qas_chunk_attention (written here from
# that text, not taken from the library or its staging helpers): blocks of 64
# lanes x 16 bytes, lane l = row + 32 * hf.
def _k_byte(t, d):
    tau, row = t // 32, t % 32
    ks, hf, c, e = d // 64, (d // 32) % 2, (d // 16) % 2, d % 16
    return (((tau * 2 + ks) * 2 + c) * 64 + row + 32 * hf) * 16 + e


def _v_byte(t, d, S):
    w, tau = t % 32, t // 32
    slot = (S // 2) * ((w // 4) % 2) + 16 * tau + 4 * (w // 8) + w % 4
    hf, rem = divmod(slot, S // 2)
    c, e = divmod(rem, 16)
    dt, row = divmod(d, 32)
    return ((dt * (S // 32) + c) * 64 + row + 32 * hf) * 16 + e


_MAPS = {}


def _token_major(tile, S, kind):
    """[S*128] stored bytes of one tile -> [S][128] codes by token and dim."""
    if (S, kind) not in _MAPS:
        _MAPS[S, kind] = np.array([[_k_byte(t, d) if kind == "k" else _v_byte(t, d, S)
                                    for d in range(128)] for t in range(S)])
    idx = _MAPS[S, kind]
    assert len(np.unique(idx)) == S * 128            # the layout is a permutation
    return tile[idx]


_IN_DTYPES = (torch.float32, torch.bfloat16, torch.float16)


def _write_in_steps(qas, case, steps, S, device="cuda"):
    """Append a request's tokens in the given chunk sizes (one request)."""
    from query_aware_sparse_amd.staging import DeviceBatch
    H = case.H_kv
    pool = case.num_pool_pages
    k_pool = torch.full((pool, H, S, 128), 0x7F, dtype=torch.uint8, device=device)
    v_pool = torch.full((pool, H, S, 128), 0x7F, dtype=torch.uint8, device=device)
    k_scale = torch.from_numpy(np.asarray(case.k_scale, np.float32)).to(device)
    v_scale = torch.from_numpy(np.asarray(case.v_scale, np.float32)).to(device)
    cache = qas.make_cache(k_pool.view(torch.float8_e4m3fn), v_pool.view(torch.float8_e4m3fn),
                           None, k_scale, v_scale)
    full = DeviceBatch([case.L], [case.pages], S, device)
    L0 = 0
    for i, n in enumerate(steps):
        before = DeviceBatch([L0], [case.pages], S, device)
        batch = qas.make_batch(before.seq_lens, full.page_indptr, full.page_indices,
                               full.total_pages, full.max_pages)
        dt = _IN_DTYPES[i % 3]                              # every input dtype
        k = torch.from_numpy(case.keys_src[L0:L0 + n].astype(np.float32)).to(device).to(dt)
        v = torch.from_numpy(case.values_src[L0:L0 + n].astype(np.float32)).to(device).to(dt)
        qas.qas_append_fp8(cache, batch, torch.tensor([0, n], dtype=torch.int32, device=device),
                           n, n, k, v)
        torch.cuda.synchronize()
        L0 += n
    assert L0 == case.L
    return k_pool.cpu().numpy(), v_pool.cpu().numpy()


def _inputs_as_written(x, steps):
    """The K/V values each step handed to the writer, as float32 (steps in
    bf16 / f16 were cast with round to nearest even by torch)."""
    out, L0 = [], 0
    for i, n in enumerate(steps):
        part = torch.from_numpy(x[L0:L0 + n].astype(np.float32)).to(_IN_DTYPES[i % 3])
        out.append(part.float().numpy())
        L0 += n
    return np.concatenate(out)


@pytest.mark.parametrize("S,steps", [(64, [100, 1, 1, 27, 1, 64, 5]),
                                     (32, [31, 1, 1, 1, 70, 33, 3])])
def test_fp8_writer_codes_equal_the_oracle(qas, S, steps):
    L = sum(steps)
    case = multiquery_chunk(seed=70 + S, L=L, S=S, N=4, H_q=8, H_kv=2, kq=4, keep=2)
    say(f"[fp8 writer] S={S} steps={steps} L={L}")
    kp, vp = _write_in_steps(qas, case, steps, S)
    for name, pool, src, scale in (("k", kp, case.keys_src, case.k_scale),
                                   ("v", vp, case.values_src, case.v_scale)):
        ref = quest.quantize_kv_e4m3(_inputs_as_written(src, steps), scale)   # [L][H][128]
        P = -(-L // S)
        for j in range(P):
            phys = case.pages[j]
            for h in range(case.H_kv):
                tile = _token_major(pool[phys, h].reshape(-1), S, name)
                n = min(S, L - j * S)
                got_vals = oracle.formats.decode_e4m3fn(tile[:n])
                ref_vals = oracle.formats.decode_e4m3fn(ref[j * S:j * S + n, h])
                assert np.array_equal(got_vals, ref_vals), f"{name} page {j} head {h}"
                # rows past the sequence in its last page hold zero codes
                assert not tile[n:].any(), f"{name} page {j} head {h}: rows past L"
        # pages outside the request's table are untouched
        used = set(int(p) for p in case.pages[:P])
        for p in range(pool.shape[0]):
            if p not in used:
                assert (pool[p] == 0x7F).all()


def test_library_cache_equals_host_placed_codes(qas):
    """Two requests sharing one pool and one pair of scales: the library's
    pools equal those placed from the workload's own e4m3 codes (torch's
    round-to-nearest cast of the same float32 quotients)."""
    from query_aware_sparse_amd.staging import ChunkBatch
    a = multiquery_chunk(seed=41, L=6000, N=21)
    b = multiquery_chunk(seed=42, L=9000, N=13, scales=(a.k_scale, a.v_scale))
    lib = ChunkBatch([a, b], writer="library")
    host = ChunkBatch([a, b], writer="host")
    torch.cuda.synchronize()
    assert torch.equal(lib.k_pool, host.k_pool)
    assert torch.equal(lib.v_pool, host.v_pool)
