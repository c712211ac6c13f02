"""Pools past 4 GiB: block ids whose byte offsets leave the 32-bit range.

Spare blocks worth 12 GiB make a pool of about 13 GB, so a random placement
puts about two thirds of a batch's blocks above 4 GiB.
Through the C ABI: the write kernel places every token (checked by decode
and prefill against the oracle), decode on the MFMA, VALU and float32 paths,
both prefill kernels, and a copy-on-write block copy between two blocks past
4 GiB (bit-exact).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import workloads as W  # noqa: E402
from tests import gpu_util as U  # noqa: E402
from oracle import attention as A  # noqa: E402
from paged_kv_cache_337_amd import staging as S  # noqa: E402

ELEM = {"f32": 4, "f16": 2, "bf16": 2}


def spare(dtype, hkv, d, bs=16):
    """Unreferenced blocks worth 12 GiB."""
    return 3 * 2 ** 32 // (2 * bs * hkv * d * ELEM[dtype])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import paged_kv_cache_337_amd  # noqa: F401


def _block_bytes(w):
    return 2 * w.block_size * w.num_kv_heads * w.head_dim * ELEM[w.dtype]


def _beyond_4gib(w):
    used = w.block_tables[w.block_tables >= 0].astype(np.int64)
    return int((used * _block_bytes(w) >= 2 ** 32).sum()), used.size


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f16", 8, 8, 128), ("f32", 8, 8, 64)])
def test_decode_beyond_4gib(dtype, hq, hkv, d):
    w = W.custom("big", 90, dtype, [3, 300, 1000, 2047], hq, hkv, d, 16, extra_blocks=spare(dtype, hkv, d))
    high, used = _beyond_4gib(w)
    U.log(f"[large] decode {dtype} G={hq // hkv}: {w.num_blocks} blocks, {high}/{used} used past 4 GiB")
    assert high > used // 2
    pool = U.make_pool(w)
    U.fill_pool(pool, w)
    q, t, c = U.device_inputs(w)
    got = U.out_f64(U.run_decode(pool, w, q, t, c))
    U.check_close(got, U.oracle_rows(w, range(w.num_seqs)), dtype, "decode, pool past 4 GiB")
    # split-K over 64-token partitions (many items, the deep schedule)
    got = U.out_f64(U.run_decode(pool, w, q, t, c, partition_tokens=64))
    U.check_close(got, U.oracle_rows(w, range(w.num_seqs)), dtype, "decode P=64, pool past 4 GiB")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_beyond_4gib(dtype):
    w = W.custom_prefill("bigp", 91, dtype, [300, 1000, 45], [300, 64, 45], 8, 2, 128, 16,
                         extra_blocks=spare(dtype, 2, 128))
    high, used = _beyond_4gib(w)
    U.log(f"[large] prefill {dtype}: {w.num_blocks} blocks, {high}/{used} used past 4 GiB")
    assert high > used // 2
    pool = U.make_pool(w)
    U.fill_pool(pool, w)
    q, qs, t, c = S.prefill_inputs(w)
    out = pool.prefill(0, q, qs, w.max_query_len, t, c, w.max_context_len, w.scale)
    torch.cuda.synchronize()
    got = U.out_f64(out)
    ref = []
    for i in range(w.num_seqs):
        K, V = w.seq_kv(i)
        qi = A.to_f64(w.q[w.query_start[i]:w.query_start[i + 1]], w.dtype)
        ref.append(A.prefill_one(qi, A.to_f64(K, w.dtype), A.to_f64(V, w.dtype), w.scale))
    U.check_close(got, np.concatenate(ref), dtype, "prefill, pool past 4 GiB")


def test_copy_blocks_beyond_4gib():
    w = W.custom("bigc", 92, "bf16", [100], 32, 8, 128, 16, extra_blocks=spare("bf16", 8, 128))
    pool = U.make_pool(w)
    U.fill_pool(pool, w)
    bb = _block_bytes(w)
    src = int(w.block_tables[0, 0])
    dst = w.num_blocks - 1  # the last block of the pool, never referenced
    if src == dst or src * bb < 2 ** 32:  # pick a referenced block past 4 GiB
        src = int(max(b for b in w.block_tables[0] if b >= 0))
    assert src * bb >= 2 ** 32 and dst * bb >= 2 ** 32 and dst not in set(w.block_tables[0].tolist())
    buf = pool.buf.view(torch.uint8)
    before = buf[dst * bb:(dst + 1) * bb].cpu()
    pool.copy_blocks(torch.tensor([[src, dst]], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    a = buf[src * bb:(src + 1) * bb].cpu()
    b = buf[dst * bb:(dst + 1) * bb].cpu()
    assert torch.equal(a, b) and not torch.equal(before, b)
