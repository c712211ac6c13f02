"""Pins of the oracle's causal prefill (new tokens attending to the cached
context and to each other) against facts fixed outside it: a library causal
attention routine on whole prompts, the decode oracle for a single new token,
exactness of the first prompt token, a 50-digit brute force, and the tail of a
whole prompt for a chunk.  ``test_planted_prefill_mistakes_are_caught`` plants
plausible slips (an off-by-one mask, positions counted from the front, no mask)
and checks that one of the pins fails."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import layout as LY
from tests.test_oracle_pins import _mp_reference, _pool_for


def _dense(w, i):
    a, b = int(w.query_start[i]), int(w.query_start[i + 1])
    K, V = w.seq_kv(i)
    return A.to_f64(w.q[a:b], w.dtype), A.to_f64(K, w.dtype), A.to_f64(V, w.dtype)


def _sdpa_causal(q, K, V, scale):
    """Whole-prompt causal attention by torch's routine: q [T, Hq, D], K/V [T, Hkv, D]."""
    import torch
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2))).unsqueeze(0)
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2))).unsqueeze(0)
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2))).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=True, scale=float(np.float32(scale)), enable_gqa=True)
    return o[0].numpy().transpose(1, 0, 2)


WHOLE_PROMPTS = [
    lambda: W.custom_prefill("p_f32", 61, "f32", [1, 7, 40], [1, 7, 40], 4, 2, 64, 16),
    lambda: W.custom_prefill("p_bf16_g4", 62, "bf16", [3, 33, 90], [3, 33, 90], 8, 2, 128, 16),
    lambda: W.custom_prefill("p_f16_g8", 63, "f16", [17, 64], [17, 64], 8, 1, 32, 32, kv_std=0.5),
    lambda: W.custom_prefill("p_mha", 64, "f16", [50], [50], 3, 3, 64, 16),
]


@pytest.mark.parametrize("mk", WHOLE_PROMPTS)
def test_whole_prompt_matches_library_causal_attention(mk):
    w = mk()
    g, pool = _pool_for(w)
    got = A.paged_prefill(pool, g, 0, w.q, w.query_start, w.block_tables, w.context_lens, w.scale)
    for i in range(w.num_seqs):
        q, K, V = _dense(w, i)
        assert np.max(np.abs(got[i] - _sdpa_causal(q, K, V, w.scale))) <= 1e-12


def test_chunk_equals_tail_of_whole_prompt():
    """n new tokens after T - n cached ones give the last n rows of the whole
    prompt's prefill over the same tokens (bit for bit)."""
    w = W.custom_prefill("chunk", 65, "bf16", [40, 77, 129], [5, 16, 33], 8, 2, 64, 16)
    for i in range(w.num_seqs):
        q, K, V = _dense(w, i)
        T, n = K.shape[0], q.shape[0]
        rng = np.random.default_rng(i)
        head = A.to_f64(W.round_to_storage(rng.standard_normal((T - n,) + q.shape[1:], dtype=np.float32),
                                           "bf16"), "bf16")
        full = np.concatenate([head, q])
        whole = A.prefill_one(full, K, V, w.scale)
        assert np.array_equal(A.prefill_one(q, K, V, w.scale), whole[T - n:])
        assert np.max(np.abs(whole - _sdpa_causal(full, K, V, w.scale))) <= 1e-12


def test_single_new_token_equals_decode():
    w = W.custom_prefill("one", 66, "f16", [1, 30, 200], [1, 1, 1], 16, 1, 64, 16)
    g, pool = _pool_for(w)
    got = A.paged_prefill(pool, g, 0, w.q, w.query_start, w.block_tables, w.context_lens, w.scale)
    dec = A.paged_decode(pool, g, 0, w.q, w.block_tables, w.context_lens, w.scale)
    for i in range(w.num_seqs):
        assert np.array_equal(got[i][0], dec[i])


def test_first_prompt_token_returns_v0_exactly():
    w = W.custom_prefill("first", 67, "bf16", [5, 40], [5, 40], 8, 2, 128, 16)
    g, pool = _pool_for(w)
    got = A.paged_prefill(pool, g, 0, w.q, w.query_start, w.block_tables, w.context_lens, w.scale)
    for i in range(w.num_seqs):
        _, V = w.seq_kv(i)
        v0 = np.repeat(A.to_f64(V[0], w.dtype), 4, axis=0)
        assert np.array_equal(got[i][0], v0)


def test_prefill_matches_brute_force():
    w = W.prefill_tiny()
    g, pool = _pool_for(w)
    rows = {0: [0, 6], 1: [0, 4], 2: [0], 3: [0, 19]}
    got = A.paged_prefill(pool, g, 0, w.q, w.query_start, w.block_tables, w.context_lens, w.scale,
                          rows=rows)
    for i in range(w.num_seqs):
        q, K, V = _dense(w, i)
        T, n = K.shape[0], q.shape[0]
        for r, k in enumerate(rows[i]):
            pos = T - n + k
            ref = _mp_reference(q[k], K[:pos + 1], V[:pos + 1], w.scale)
            assert np.max(np.abs(got[i][r] - ref)) <= 1e-12


def test_paged_prefill_equals_dense_and_ignores_placement():
    w = W.custom_prefill("place", 68, "f16", [3, 16, 40, 77], [3, 4, 17, 1], 8, 2, 64, 16, extra_blocks=6)
    g, pool = _pool_for(w)
    got = A.paged_prefill(pool, g, 0, w.q, w.query_start, w.block_tables, w.context_lens, w.scale)
    for i in range(w.num_seqs):
        assert np.array_equal(got[i], A.prefill_one(*_dense(w, i), w.scale))
    # relabel physical blocks
    pi = np.random.default_rng(1).permutation(w.num_blocks)
    region = 2 * g.bs * g.D * g.H
    pool2 = np.empty_like(pool)
    pool2.reshape(w.num_blocks, region)[pi] = pool.reshape(w.num_blocks, region)
    tables2 = np.where(w.block_tables >= 0, pi[np.maximum(w.block_tables, 0)], -1)
    got2 = A.paged_prefill(pool2, g, 0, w.q, w.query_start, tables2, w.context_lens, w.scale)
    for a, b in zip(got, got2):
        assert np.array_equal(a, b)


def test_prefill_rejects_bad_lengths():
    q = np.zeros((3, 2, 8))
    K = np.zeros((2, 1, 8))
    with pytest.raises(ValueError):
        A.prefill_one(q, K, K, 1.0)
    with pytest.raises(ValueError):
        A.prefill_one(q[:0], K, K, 1.0)
    with pytest.raises(ValueError):
        W.custom_prefill("bad", 1, "f32", [4], [5], 2, 2, 64, 16)


def test_prefill_generator_self_check_values():
    w = W.prefill_llama3_8b()
    assert w.total_tokens == int(w.query_lens.sum()) == 21_256
    c = W.chunked_llama3_8b()
    assert c.total_tokens == 106_925 and int(c.query_lens.sum()) == 16_384
    assert W.prefill_tiny().query_start.tolist() == [0, 7, 12, 13, 33]


# ------------------------------------------------------- planted mistakes ---

def _mutants():
    def off_by_one_mask(q, K, V, s):
        n, T = q.shape[0], K.shape[0]
        return np.stack([A.decode_one(q[k], K[:max(T - n + k, 1)], V[:max(T - n + k, 1)], s)
                         for k in range(n)])

    def positions_from_front(q, K, V, s):
        return np.stack([A.decode_one(q[k], K[:k + 1], V[:k + 1], s) for k in range(q.shape[0])])

    def no_mask(q, K, V, s):
        return np.stack([A.decode_one(q[k], K, V, s) for k in range(q.shape[0])])

    def mask_one_too_far(q, K, V, s):
        n, T = q.shape[0], K.shape[0]
        return np.stack([A.decode_one(q[k], K[:min(T - n + k + 2, T)], V[:min(T - n + k + 2, T)], s)
                         for k in range(n)])

    return [off_by_one_mask, positions_from_front, no_mask, mask_one_too_far]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_prefill_mistakes_are_caught(mutant):
    """Each slip fails the whole-prompt library pin or the chunk-tail pin."""
    w = W.custom_prefill("mut", 69, "bf16", [20, 45], [20, 9], 8, 2, 32, 16)
    caught = False
    # whole prompt vs the library routine
    q, K, V = _dense(w, 0)
    if np.max(np.abs(mutant(q, K, V, w.scale) - _sdpa_causal(q, K, V, w.scale))) > 1e-6:
        caught = True
    # chunk vs the tail of the whole prompt over the same tokens
    q, K, V = _dense(w, 1)
    T, n = K.shape[0], q.shape[0]
    head = np.zeros((T - n,) + q.shape[1:])
    full = np.concatenate([head, q])
    if not np.array_equal(mutant(q, K, V, w.scale), mutant(full, K, V, w.scale)[T - n:]):
        caught = True
    assert caught
