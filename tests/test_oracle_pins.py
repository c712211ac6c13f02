"""Pins of the CPU oracle against facts fixed outside it: values the pages
print, closed forms, a 50-digit brute force, a library attention routine, and
invariances of attention.  Each pin is chosen so that a plausible slip in the
oracle (a dropped term or token, a wrong index or grouping, a sign) fails it;
``test_planted_mistakes_are_caught`` checks exactly that."""
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import layout as LY
from oracle import sizing as SZ

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


# ---------------------------------------------------------------- sizing ---

def test_block_counts_match_pages():
    for tok, bs, blocks, unused in _rows("block_counts.txt"):
        assert SZ.blocks_required(int(tok), int(bs)) == int(blocks)
        assert SZ.unused_slots(int(tok), int(bs)) == int(unused)


def test_block_count_error_rules():
    with pytest.raises(ValueError):
        SZ.blocks_required(-1, 16)
    with pytest.raises(ValueError):
        SZ.blocks_required(10, 0)
    with pytest.raises(ValueError):
        SZ.blocks_required(10, -16)
    assert SZ.blocks_required(0, 16) == 0


def test_pool_bytes_closed_form():
    # 2 * L * T * H_kv * D * B with T = N * bs slots
    for L, N, bs, H, D, dt in [(1, 32, 16, 4, 64, "f32"), (2, 7, 32, 8, 128, "bf16"),
                               (3, 5, 16, 40, 128, "f16")]:
        g = LY.Geometry(L, N, bs, H, D, dt)
        B = LY.ITEMSIZE[dt]
        assert g.num_elements * B == SZ.pool_bytes(L, N, bs, H, D, B) == 2 * L * N * bs * H * D * B
    w = W.opt13b()
    assert SZ.pool_bytes(1, w.num_blocks, 16, 40, 128, 2) == 1_514_864_640


def test_generator_self_check_values():
    assert W.opt13b().total_tokens == 73_505
    assert W.llama3_8b().total_tokens == 366_900
    assert W.long_ctx().total_tokens == 854_921
    assert W.tiny().context_lens.tolist() == [7, 16, 33, 50]


# ---------------------------------------------------------------- layout ---

@pytest.mark.parametrize("geom", [(1, 3, 16, 2, 64, "f32"), (2, 3, 32, 2, 128, "bf16"),
                                  (1, 2, 16, 3, 64, "f16"), (1, 2, 48, 1, 32, "bf16")])
def test_layout_is_a_bijection(geom):
    g = LY.Geometry(*geom)
    L, N, H, kv, t, d = np.meshgrid(np.arange(g.L), np.arange(g.N), np.arange(g.H), np.arange(2),
                                    np.arange(g.bs), np.arange(g.D), indexing="ij")
    idx = LY.element_index(g, L, N, H, kv, t, d).ravel()
    assert np.array_equal(np.sort(idx), np.arange(g.num_elements))
    # each (layer, block, head) owns one contiguous region of 2*bs*D elements
    region = idx // (2 * g.bs * g.D)
    assert np.array_equal(region, (((L * g.N + N) * g.H + H)).ravel())


def test_mapping_example_from_pages():
    rows = _rows("mapping_example.txt")
    bs = int(rows[0][0])
    table = np.array([int(x) for x in rows[1]], dtype=np.int32)
    g = LY.Geometry(1, 13, bs, 2, 64, "f32")
    ik, iv = LY.token_indices(g, 0, table, 3 * bs)
    region = 2 * bs * g.D * g.H
    for p in range(3 * bs):
        assert np.all(ik[p] // region == table[p // bs])
        assert np.all(iv[p] // region == table[p // bs])
    # slot numbering block*bs + offset: position 0 -> block 7, 16 -> block 3, 39 -> block 12
    assert [LY.slot_of(table, bs, p) for p in (0, 15, 16, 20, 39)] == [112, 127, 48, 52, 199]


def test_scatter_gather_round_trip():
    w = W.custom("rt", 11, "bf16", [5, 16, 17, 40], 8, 2, 128, 32, extra_blocks=3)
    g = LY.Geometry(2, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
    pool = np.full(g.num_elements, W.POISON_BITS["bf16"], dtype=np.uint16)
    for i in range(w.num_seqs):
        K, V = w.seq_kv(i)
        LY.scatter(pool, g, 1, w.block_tables[i], K, V)
    for i in range(w.num_seqs):
        K, V = w.seq_kv(i)
        K2, V2 = LY.gather(pool, g, 1, w.block_tables[i], int(w.context_lens[i]))
        assert np.array_equal(K, K2) and np.array_equal(V, V2)
    # layer 0 untouched
    assert np.all(pool[: g.num_elements // 2] == W.POISON_BITS["bf16"])


# ------------------------------------------------------------- attention ---

def _pool_for(w, layers=1, layer=0):
    g = LY.Geometry(layers, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype)
    pool = np.full(g.num_elements, W.POISON_BITS[w.dtype], dtype=W.storage_numpy_dtype(w.dtype)) \
        if w.dtype == "bf16" else np.full(g.num_elements, np.nan, dtype=W.storage_numpy_dtype(w.dtype))
    for i in range(w.num_seqs):
        K, V = w.seq_kv(i)
        LY.scatter(pool, g, layer, w.block_tables[i], K, V)
    return g, pool


def _mp_reference(q, K, V, scale):
    """Per-token loop in 50-digit arithmetic."""
    import mpmath as mp
    mp.mp.dps = 50
    Hq, D = q.shape
    T, Hkv, _ = K.shape
    G = Hq // Hkv
    sigma = mp.mpf(float(np.float32(scale)))
    out = np.empty((Hq, D))
    for g in range(Hq):
        h = g // G
        s = [sigma * mp.fsum(mp.mpf(float(q[g, d])) * mp.mpf(float(K[p, h, d])) for d in range(D))
             for p in range(T)]
        m = max(s)
        e = [mp.e ** (x - m) for x in s]
        l = mp.fsum(e)
        for d in range(D):
            out[g, d] = float(mp.fsum(e[p] * mp.mpf(float(V[p, h, d])) for p in range(T)) / l)
    return out


SMALL = [
    lambda: W.tiny(),
    lambda: W.custom("gqa", 21, "bf16", [1, 3, 17], 4, 2, 32, 16),
    lambda: W.custom("gqa8", 22, "f16", [9, 33], 8, 1, 32, 32, kv_std=0.5),
]


@pytest.mark.parametrize("mk", SMALL)
def test_oracle_matches_brute_force(mk):
    w = mk()
    g, pool = _pool_for(w)
    seqs = range(w.num_seqs) if w.name != "tiny" else [0, 3]
    got = A.paged_decode(pool, g, 0, w.q, w.block_tables, w.context_lens, w.scale, seqs=seqs)
    for n, i in enumerate(seqs):
        K, V = w.seq_kv(i)
        ref = _mp_reference(A.to_f64(w.q[i], w.dtype), A.to_f64(K, w.dtype), A.to_f64(V, w.dtype), w.scale)
        assert np.max(np.abs(got[n] - ref)) <= 1e-12


def _sdpa(q, K, V, scale):
    import torch
    qt = torch.from_numpy(q)[:, None, :].unsqueeze(0)          # [1, Hq, 1, D]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2))).unsqueeze(0)  # [1, Hkv, T, D]
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2))).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, scale=float(np.float32(scale)), enable_gqa=True)
    return o[0, :, 0, :].numpy()


@pytest.mark.parametrize("mk", SMALL + [lambda: W.scaled_down(W.llama3_8b(), 6, 300),
                                        lambda: W.scaled_down(W.long_ctx(), 2, 700)])
def test_oracle_matches_library_attention(mk):
    w = mk()
    g, pool = _pool_for(w)
    got = A.paged_decode(pool, g, 0, w.q, w.block_tables, w.context_lens, w.scale)
    for i in range(w.num_seqs):
        K, V = w.seq_kv(i)
        ref = _sdpa(A.to_f64(w.q[i], w.dtype), A.to_f64(K, w.dtype), A.to_f64(V, w.dtype), w.scale)
        assert np.max(np.abs(got[i] - ref)) <= 1e-12


def test_hand_worked_closed_form():
    exp = np.array([float(x) for x in _rows("hand_worked.txt")[0]])
    q = np.array([[math.log(3.0), 0.0]])
    K = np.array([[[1.0, 0.0]], [[0.0, 0.0]]])
    V = np.array([[[4.0, 0.0]], [[0.0, 8.0]]])
    o = A.decode_one(q, K, V, 1.0)
    assert np.max(np.abs(o[0] - exp)) <= 1e-12


def test_identity_table_equals_dense_attention():
    w = W.scaled_down(W.llama3_8b(), 5, 200)
    g, pool = _pool_for(w)
    paged = A.paged_decode(pool, g, 0, w.q, w.block_tables, w.context_lens, w.scale)
    # contiguous layout: blocks of each sequence in logical order 0, 1, 2, ...
    ident = np.full_like(w.block_tables, -1)
    off = 0
    for i, c in enumerate(w.context_lens):
        n = SZ.blocks_required(int(c), w.block_size)
        ident[i, :n] = np.arange(off, off + n)
        off += n
    w2 = W.PagedWorkload(**{**w.__dict__, "block_tables": ident})
    g2, pool2 = _pool_for(w2)
    contig = A.paged_decode(pool2, g2, 0, w.q, ident, w.context_lens, w.scale)
    dense = np.stack([A.decode_one(A.to_f64(w.q[i], w.dtype), *(A.to_f64(x, w.dtype) for x in w.seq_kv(i)),
                                   w.scale) for i in range(w.num_seqs)])
    assert np.array_equal(paged, dense) and np.array_equal(contig, dense)


def test_physical_relabeling_is_bit_identical():
    w = W.custom("relabel", 31, "f16", [3, 16, 40, 77], 8, 2, 64, 16, extra_blocks=5)
    g, pool = _pool_for(w)
    ref = A.paged_decode(pool, g, 0, w.q, w.block_tables, w.context_lens, w.scale)
    pi = np.random.default_rng(0).permutation(w.num_blocks)
    pool2 = np.empty_like(pool)
    region = 2 * g.bs * g.D * g.H
    pr = pool.reshape(w.num_blocks, region)
    pool2.reshape(w.num_blocks, region)[pi] = pr
    tables2 = np.where(w.block_tables >= 0, pi[np.maximum(w.block_tables, 0)], -1)
    got = A.paged_decode(pool2, g, 0, w.q, tables2, w.context_lens, w.scale)
    assert np.array_equal(ref, got)


def test_single_token_context_returns_v_exactly():
    w = W.custom("ctx1", 41, "bf16", [1, 1, 1], 8, 2, 128, 16)
    g, pool = _pool_for(w)
    got = A.paged_decode(pool, g, 0, w.q, w.block_tables, w.context_lens, w.scale)
    for i in range(3):
        _, V = w.seq_kv(i)
        v = A.to_f64(V[0], w.dtype)
        assert np.array_equal(got[i], np.repeat(v, 4, axis=0))


def test_zero_query_returns_mean_of_v():
    w = W.custom("q0", 42, "f32", [5, 50, 129], 4, 4, 64, 16)
    w.q[:] = 0
    g, pool = _pool_for(w)
    got = A.paged_decode(pool, g, 0, w.q, w.block_tables, w.context_lens, w.scale)
    for i in range(3):
        _, V = w.seq_kv(i)
        mean = A.to_f64(V, w.dtype).mean(axis=0)
        assert np.max(np.abs(got[i] - mean)) <= 1e-15 * max(1, int(w.context_lens[i]))


def test_v_shift_shifts_output():
    w = W.custom("vs", 43, "f32", [9, 70], 4, 2, 64, 16)
    c = 3.25
    for i in range(2):
        K, V = w.seq_kv(i)
        q, Kf, Vf = A.to_f64(w.q[i], "f32"), A.to_f64(K, "f32"), A.to_f64(V, "f32")
        a = A.decode_one(q, Kf, Vf, w.scale)
        b = A.decode_one(q, Kf, Vf + c, w.scale)
        assert np.max(np.abs(b - a - c)) <= 1e-12


@pytest.mark.parametrize("P", [1, 16, 37, 512, 4096])
def test_split_k_merge_equals_unsplit(P):
    w = W.custom("split", 44, "bf16", [1, 600, 1300], 8, 1, 64, 32, kv_std=0.5)
    for i in range(w.num_seqs):
        K, V = w.seq_kv(i)
        q, Kf, Vf = A.to_f64(w.q[i], "bf16"), A.to_f64(K, "bf16"), A.to_f64(V, "bf16")
        assert np.max(np.abs(A.split_decode(q, Kf, Vf, w.scale, P) - A.decode_one(q, Kf, Vf, w.scale))) <= 1e-12


def test_gather_rejects_bad_tables_and_empty_context():
    w = W.tiny()
    g, pool = _pool_for(w)
    with pytest.raises(ValueError):
        LY.gather(pool, g, 0, w.block_tables[0], 0)
    bad = w.block_tables[3].copy()
    bad[1] = -1
    with pytest.raises(ValueError):
        LY.gather(pool, g, 0, bad, 50)


# ------------------------------------------------------- planted mistakes ---

def _mutant_decodes():
    def drop_last_token(q, K, V, s):
        return A.decode_one(q, K[:-1], V[:-1], s) if K.shape[0] > 1 else A.decode_one(q, K, V, s) * 0

    def wrong_grouping(q, K, V, s):
        Hq, Hkv = q.shape[0], K.shape[1]
        out = np.empty_like(q)
        for g in range(Hq):
            out[g] = A.decode_one(q[g:g + 1], K[:, [g % Hkv]], V[:, [g % Hkv]], s)[0]
        return out

    def sign_flip(q, K, V, s):
        return A.decode_one(-q, K, V, s)

    def no_scale(q, K, V, s):
        return A.decode_one(q, K, V, 1.0)

    def transposed_v(q, K, V, s):
        return A.decode_one(q, K, V[::-1], s)

    return [drop_last_token, wrong_grouping, sign_flip, no_scale, transposed_v]


@pytest.mark.parametrize("mutant", _mutant_decodes(), ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught(mutant):
    """Each planted slip must be caught by the library-routine pin on a GQA case."""
    w = W.custom("mut", 51, "bf16", [3, 17, 40], 8, 2, 32, 16)
    caught = False
    for i in range(w.num_seqs):
        K, V = w.seq_kv(i)
        q, Kf, Vf = A.to_f64(w.q[i], "bf16"), A.to_f64(K, "bf16"), A.to_f64(V, "bf16")
        if np.max(np.abs(mutant(q, Kf, Vf, w.scale) - _sdpa(q, Kf, Vf, w.scale))) > 1e-6:
            caught = True
    assert caught


def test_staged_lse_merge_equals_unsplit():
    """Split-K over fixed partitions, combined in two stages: four neighbouring
    partition states into a group state (max M, sum L relative to M, output),
    then the group states.  The log-sum-exp combination is associative, so the
    staged result is the unsplit attention to rounding; carrying a group's sum
    wrongly (L = 1) is caught."""
    rng = np.random.default_rng(11)
    for T, P in [(1, 16), (100, 16), (1000, 64), (2049, 512), (5000, 512)]:
        q = rng.standard_normal((8, 32))
        K = rng.standard_normal((T, 2, 32)) * 2.0
        V = rng.standard_normal((T, 2, 32))
        states = [A.partition_state(q, K[a:a + P], V[a:a + P], 0.17) for a in range(0, T, P)]

        def staged(carry_sum=True):
            groups = []
            for g0 in range(0, len(states), 4):
                grp = states[g0:g0 + 4]
                ms = np.array([st[0] for st in grp])
                ls = np.array([st[1] for st in grp])
                M = ms.max(axis=0)
                L = (ls * np.exp(ms - M)).sum(axis=0) if carry_sum else np.ones_like(M)
                groups.append((M, L, A.lse_merge(ms, ls, [st[2] for st in grp])))
            return A.lse_merge([g[0] for g in groups], [g[1] for g in groups], [g[2] for g in groups])

        ref = A.decode_one(q, K, V, 0.17)
        assert np.max(np.abs(staged() - ref)) <= 1e-12, (T, P)
        if len(states) > 4:  # two or more groups: the group sums matter
            assert np.max(np.abs(staged(carry_sum=False) - ref)) > 1e-6, (T, P)


# --------------------------------------------------- storage widening -------
#
# Every other attention pin feeds its inputs through ``A.to_f64``, so a slip
# there (a wrong shift, a lost sign bit, the wrong half of the word) would pass
# them all.  These pins fix the widening from outside the oracle: bfloat16 is
# the upper 16 bits of an IEEE-754 binary32 (1 sign, 8 exponent, 7 fraction
# bits), binary16 has 1/5/10 bits; the values below follow from those formats
# alone, and the exhaustive check compares with torch's own bfloat16 type.

def _bf16_fixed_points():
    return [
        (0x3F80, 1.0), (0xBF80, -1.0), (0xC000, -2.0), (0x4049, 3.140625),
        (0x3F81, 1.0 + 2.0 ** -7), (0x0080, 2.0 ** -126),           # smallest normal
        (0x0001, 2.0 ** -133), (0x8001, -(2.0 ** -133)),            # smallest subnormal
        (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),                   # largest finite
        (0x7F80, math.inf), (0xFF80, -math.inf), (0x0000, 0.0),
    ]


def _f16_fixed_points():
    return [
        (0x3C00, 1.0), (0xC000, -2.0), (0x0001, 2.0 ** -24), (0x0400, 2.0 ** -14),
        (0x7BFF, 65504.0), (0x3555, 0.333251953125), (0xFC00, -math.inf),
    ]


def _widening_failures(fn):
    """Names of the widening pins that ``fn(bits_or_values, dtype)`` fails."""
    import torch
    bad = []
    bits = np.array([b for b, _ in _bf16_fixed_points()], dtype=np.uint16)
    want = np.array([v for _, v in _bf16_fixed_points()])
    got = fn(bits, "bf16")
    if got.dtype != np.float64 or not np.array_equal(got, want):
        bad.append("bf16 fixed points")
    # -0.0 keeps its sign
    if not np.signbit(fn(np.array([0x8000], dtype=np.uint16), "bf16")[0]):
        bad.append("bf16 negative zero")
    # every bf16 pattern against torch's bfloat16 -> float64 conversion
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(allb.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    with np.errstate(invalid="ignore"):
        got = fn(allb, "bf16")
    nan = np.isnan(ref)
    if not (np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], ref[~nan])):
        bad.append("bf16 exhaustive")
    hb = np.array([b for b, _ in _f16_fixed_points()], dtype=np.uint16)
    hv = np.array([v for _, v in _f16_fixed_points()])
    if not np.array_equal(fn(hb.view(np.float16), "f16"), hv):
        bad.append("f16 fixed points")
    f32 = np.array([1.0, -2.5, 2.0 ** -149, 3.4028234663852886e38], dtype=np.float32)
    if not np.array_equal(fn(f32, "f32"), f32.astype(np.float64)):
        bad.append("f32 identity")
    return bad


def test_storage_widening_is_exact():
    assert _widening_failures(A.to_f64) == []


def _widening_mutants():
    def shift_15(x, dt):
        if dt == "bf16":
            return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 15).view(np.float32).astype(np.float64)
        return A.to_f64(x, dt)

    def lost_sign(x, dt):
        if dt == "bf16":
            return A.to_f64(np.asarray(x, dtype=np.uint16) & np.uint16(0x7FFF), dt)
        return A.to_f64(x, dt)

    def low_half(x, dt):  # the bits placed in the low half of the word
        if dt == "bf16":
            return np.asarray(x, dtype=np.uint16).astype(np.uint32).view(np.float32).astype(np.float64)
        return A.to_f64(x, dt)

    def via_f16(x, dt):  # bf16 bits read as binary16
        if dt == "bf16":
            return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)
        return A.to_f64(x, dt)

    def rounded_f16(x, dt):  # f16 widened through a lossy path
        if dt == "f16":
            return np.asarray(x).astype(np.float64).round(3)
        return A.to_f64(x, dt)

    return [shift_15, lost_sign, low_half, via_f16, rounded_f16]


@pytest.mark.parametrize("mutant", _widening_mutants(), ids=lambda f: f.__name__)
def test_widening_slips_are_caught(mutant):
    assert _widening_failures(mutant) != []
