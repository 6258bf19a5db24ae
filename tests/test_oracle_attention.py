"""Pins of the oracle's paged attention and log-sum-exp merge.

What fixes each result independently of the oracle's own code:
  * torch's fp64 scaled_dot_product_attention over the dense gather, with its own
    GQA rule (``enable_gqa``) and its own bottom-right causal mask
    (``causal_lower_right``: query i of L sees keys up to S - L + i);
  * closed forms: constant V, zero query, single key, a dominant needle;
  * invariants: block-table permutation, split-KV partials merged == whole,
    empty rows give exactly 0 and -inf;
  * brute force with scalar Python loops on a tiny case.
The pages behind the checked behaviour: vLLM PR #50371 (test plan: fp32 SDPA
reference; padded heads leave the real heads unchanged), diffbot model card
("Update 2026-10-01": rows without visible keys give 0).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import workloads
from oracle import paged_ref as R


def spec_of(w):
    return R.CacheSpec.from_geom(w.geom)


def written_cache(w):
    """Cache bits after the workload's write (oracle write), as a flat numpy array."""
    spec = spec_of(w)
    img = w.cache_init.numpy()
    kb = w.key.view(torch.int16).numpy().view(np.uint16)
    vb = w.value.view(torch.int16).numpy().view(np.uint16) if w.value is not None else None
    if spec.kv_dtype == "fp8":
        return R.cache_write(img, spec, kb, vb, w.slot_mapping.numpy(), w.k_scale, w.v_scale)
    out = R.cache_write(img.view(np.uint16), spec, kb, vb, w.slot_mapping.numpy())
    if "pre_slots" in w.extra:
        pk = w.extra["pre_key"].view(torch.int16).numpy().view(np.uint16)
        pv = w.extra["pre_value"]
        pv = pv.view(torch.int16).numpy().view(np.uint16) if pv is not None else None
        out = R.cache_write(out, spec, pk, pv, w.extra["pre_slots"].numpy())
    return out


def run_oracle(w, cache=None, **kw):
    cache = written_cache(w) if cache is None else cache
    qb = w.q.view(torch.int16).numpy().view(np.uint16)
    return R.paged_attention(qb, w.query_start_loc.numpy(), w.seq_lens.numpy(), w.block_tables.numpy(),
                             cache, spec_of(w), w.softmax_scale, w.k_scale, w.v_scale, **kw)


def sdpa_reference(w, cache):
    """torch fp64 SDPA per sequence on the dense K/V gathered by torch indexing."""
    g = w.geom
    if g.kv_dtype == "fp8":
        vals = torch.from_numpy(cache).view(torch.float8_e4m3fn).to(torch.float64)
    else:
        vals = torch.from_numpy(cache.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    view = vals[: g.cache_elems].view(g.num_blocks, g.block_size, g.num_kv_heads, g.row_dim)
    q = w.q.to(torch.float64)
    outs = torch.zeros(q.shape[0], q.shape[1], g.head_dim_v, dtype=torch.float64)
    qsl = w.query_start_loc.tolist()
    for b, S in enumerate(w.seq_lens.tolist()):
        L = qsl[b + 1] - qsl[b]
        if S == 0 or L == 0:
            continue
        j = torch.arange(S)
        rows = view[w.block_tables[b].long()[j // g.block_size], j % g.block_size]   # [S, Hkv, W]
        K = rows[..., : g.head_dim_k]
        V = rows[..., g.v_offset: g.v_offset + g.head_dim_v]
        if w.k_scale is not None:
            ks = w.k_scale.to(torch.float64).expand(g.num_kv_heads)
            vs = w.v_scale.to(torch.float64).expand(g.num_kv_heads)
            K, V = K * ks[None, :, None], V * vs[None, :, None]
        qq = q[qsl[b]: qsl[b + 1]].transpose(0, 1)[None]        # [1, Hq, L, Dk]
        kk, vv = K.transpose(0, 1)[None], V.transpose(0, 1)[None]
        o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=causal_lower_right(L, S),
                                           scale=w.softmax_scale, enable_gqa=True)
        outs[qsl[b]: qsl[b + 1]] = o[0].transpose(0, 1)
    return outs.numpy()


def small_workload(seq_lens, query_lens, hq=8, hkv=2, bs=16, seed=1, kv_dtype="bf16", scale_mode="none",
                   dk=192, dv=128, v_off=192, row=320):
    g = workloads.CacheGeom(0, bs, hkv, dk, dv, v_off, row, kv_dtype)
    return workloads.paged_workload("small", g, seq_lens, query_lens, hq, 1 / math.sqrt(dk), seed=seed,
                                    scale_mode=scale_mode)


@pytest.mark.parametrize("case", ["tiny", "verify", "mixed", "fp8_tensor", "fp8_head", "mla"])
def test_oracle_matches_torch_sdpa(case):
    if case == "tiny":
        w = workloads.tiny()
    elif case == "verify":
        w = small_workload([45, 70], [4, 4])
    elif case == "mixed":
        w = small_workload([1, 16, 17, 33], [1, 16, 5, 2], hq=6, hkv=3, bs=8)
    elif case == "fp8_tensor":
        w = small_workload([50, 23], [4, 3], kv_dtype="fp8", scale_mode="tensor")
    elif case == "fp8_head":
        w = small_workload([50, 23], [4, 3], kv_dtype="fp8", scale_mode="head")
    else:
        w = small_workload([40, 9], [1, 2], hq=12, hkv=1, bs=16, dk=576, dv=512, v_off=0, row=576)
    cache = written_cache(w)
    out, lse = run_oracle(w, cache)
    ref = sdpa_reference(w, cache)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(3)
    S, Hkv, Hq, Dk, Dv = 29, 2, 4, 16, 8
    K = rng.standard_normal((S, Hkv, Dk))
    q = rng.standard_normal((3, Hq, Dk))
    pos = np.array([S - 3, S - 2, S - 1])
    # constant V -> output is that constant, whatever the scores
    V = np.full((S, Hkv, Dv), 0.375)
    out, _ = R.attention_rows(q, K, V, pos, 0.3)
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-15)
    # zero query -> uniform weights -> mean of the visible V rows; lse = ln(#visible)
    V = rng.standard_normal((S, Hkv, Dv))
    out, lse = R.attention_rows(np.zeros_like(q), K, V, pos, 0.3)
    for i, p in enumerate(pos):
        for h in range(Hq):
            np.testing.assert_allclose(out[i, h], V[: p + 1, h // 2].mean(axis=0), atol=1e-14)
            assert abs(lse[i, h] - math.log(p + 1)) < 1e-13
    # a single visible key -> that key's V row, lse = its score
    out, lse = R.attention_rows(q, K, V, np.array([0, 0, 0]), 0.3)
    for h in range(Hq):
        np.testing.assert_allclose(out[:, h], np.broadcast_to(V[0, h // 2], (3, Dv)), atol=1e-15)
        np.testing.assert_allclose(lse[:, h], 0.3 * (q[:, h] @ K[0, h // 2]), atol=1e-13)
    # a needle 50 nats above the rest -> its V row (to exp(-50) relative)
    Kn = np.zeros((S, Hkv, Dk))
    qn = np.zeros((1, Hq, Dk))
    qn[0, :, 0] = 1.0
    Kn[11, :, 0] = 50.0
    out, _ = R.attention_rows(qn, Kn, V, np.array([S - 1]), 1.0)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], V[11, h // 2], atol=1e-19 * S + 1e-12)


def test_brute_force_scalar_loops():
    """Scalar Python loops (math.exp) on a tiny GQA case with causal offsets."""
    w = small_workload([5, 3], [2, 3], hq=4, hkv=2, bs=4, seed=7, dk=8, dv=4, v_off=8, row=12)
    cache = written_cache(w)
    out, lse = run_oracle(w, cache)
    vals = cache.view(np.uint16).astype(np.uint32) << 16
    vals = vals.view(np.float32).astype(np.float64)
    g = w.geom
    q = w.q.to(torch.float64).numpy()
    qsl = w.query_start_loc.tolist()
    for b, S in enumerate(w.seq_lens.tolist()):
        L = qsl[b + 1] - qsl[b]
        for i in range(L):
            t = qsl[b] + i
            for h in range(w.num_q_heads):
                kvh = h // (w.num_q_heads // g.num_kv_heads)
                scores, rows = [], []
                for j in range(S - L + i + 1):
                    blk = int(w.block_tables[b, j // g.block_size])
                    base = ((blk * g.block_size + j % g.block_size) * g.num_kv_heads + kvh) * g.row_dim
                    kj = vals[base: base + g.head_dim_k]
                    scores.append(w.softmax_scale * sum(q[t, h, d] * kj[d] for d in range(g.head_dim_k)))
                    rows.append(vals[base + g.v_offset: base + g.v_offset + g.head_dim_v])
                m = max(scores)
                e = [math.exp(s - m) for s in scores]
                tot = sum(e)
                ref = [sum(e[j] * rows[j][d] for j in range(len(e))) / tot for d in range(g.head_dim_v)]
                np.testing.assert_allclose(out[t, h], ref, rtol=1e-12, atol=1e-14)
                assert abs(lse[t, h] - (m + math.log(tot))) < 1e-12


def test_block_table_permutation_invariance():
    w = workloads.tiny()
    cache = written_cache(w)
    out, lse = run_oracle(w, cache)
    # move every physical block to a new place and rewrite the tables to match
    g = w.geom
    perm = np.random.default_rng(5).permutation(g.num_blocks)
    blocks = cache[: g.cache_elems].reshape(g.num_blocks, -1)
    moved = cache.copy()
    moved[: g.cache_elems].reshape(g.num_blocks, -1)[perm] = blocks
    w2 = workloads.tiny()
    w2.block_tables = torch.from_numpy(perm[w.block_tables.numpy()].astype(np.int32))
    out2, lse2 = run_oracle(w2, moved)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_empty_rows_give_zero_and_minus_inf():
    w = small_workload([20, 0, 0], [4, 1, 1])
    out, lse = run_oracle(w)
    assert np.all(out[4:] == 0.0) and not np.any(np.signbit(out[4:]))
    assert np.all(np.isneginf(lse[4:]))
    assert np.all(np.isfinite(out[:4]))


@pytest.mark.parametrize("P", [1, 2, 3, 7, 16])
def test_partials_merge_to_whole(P):
    w = small_workload([45, 70, 0], [4, 1, 1], bs=8)
    cache = written_cache(w)
    out, lse = run_oracle(w, cache)
    qb = w.q.view(torch.int16).numpy().view(np.uint16)
    po, pl = R.paged_attention_partials(qb, w.query_start_loc.numpy(), w.seq_lens.numpy(),
                                        w.block_tables.numpy(), cache, spec_of(w), w.softmax_scale, P)
    m_out, m_lse = R.merge_lse(po, pl)
    np.testing.assert_allclose(m_out, out, rtol=0, atol=1e-12)
    fin = np.isfinite(lse)
    np.testing.assert_allclose(m_lse[fin], lse[fin], rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(m_lse), np.isneginf(lse))


def test_partition_ranges_cover_keys_once():
    for S in [0, 1, 15, 16, 17, 100, 4097, 131072]:
        for P in [1, 3, 16, 64, 96]:
            rng = R.partition_ranges(S, P, 16)
            assert len(rng) == P
            covered = [j for lo, hi in rng for j in range(lo, hi)] if S < 5000 else None
            if covered is not None:
                assert covered == list(range(S))
            assert all(lo % 16 == 0 or lo == S for lo, hi in rng)


def test_partition_ranges_closed_form():
    """The 16-key rule the library documents, independent of the block size: C = ceil(S / P)
    rounded up to 16 (values worked out by hand)."""
    assert R.partition_ranges(100, 3) == [(0, 48), (48, 96), (96, 100)]
    assert R.partition_ranges(37, 4) == [(0, 16), (16, 32), (32, 37), (37, 37)]
    r = R.partition_ranges(100000, 224)                 # 447 keys -> 448
    assert r[0] == (0, 448) and r[222] == (99456, 99904) and r[223] == (99904, 100000)
    r = R.partition_ranges(100000, 16)                  # 6250 -> 6256
    assert r[1] == (6256, 12512) and r[15] == (93840, 100000)
    r = R.partition_ranges(131072, 128)
    assert all(hi - lo == 1024 for lo, hi in r)
    assert R.partition_ranges(5, 7) == [(0, 5)] + [(5, 5)] * 6


def _sdpa_range(w, cache, b, lo, hi):
    """torch fp64 attention of sequence b's query rows over keys [lo, hi) only (explicit mask:
    key j visible to query i iff j <= S - L + i); returns out [L, Hq, Dv] and lse [L, Hq]."""
    g = w.geom
    vals = torch.from_numpy(cache.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    view = vals[: g.cache_elems].view(g.num_blocks, g.block_size, g.num_kv_heads, g.row_dim)
    qsl = w.query_start_loc.tolist()
    S, L = int(w.seq_lens[b]), qsl[b + 1] - qsl[b]
    j = torch.arange(lo, hi)
    rows = view[w.block_tables[b].long()[j // g.block_size], j % g.block_size]
    K = rows[..., : g.head_dim_k].transpose(0, 1)                         # [Hkv, n, Dk]
    V = rows[..., g.v_offset: g.v_offset + g.head_dim_v].transpose(0, 1)
    G = w.num_q_heads // g.num_kv_heads
    K, V = K.repeat_interleave(G, 0), V.repeat_interleave(G, 0)           # [Hq, n, D]
    q = w.q[qsl[b]: qsl[b + 1]].to(torch.float64).transpose(0, 1)        # [Hq, L, Dk]
    vis = j[None, :] <= (S - L + torch.arange(L))[:, None]                # [L, n]
    sc = torch.where(vis[None], torch.matmul(q, K.transpose(1, 2)) * w.softmax_scale, -torch.inf)
    lse = torch.logsumexp(sc, dim=-1)                                     # [Hq, L]
    out = torch.matmul(torch.softmax(sc, dim=-1), V)
    return out.transpose(0, 1).numpy(), lse.transpose(0, 1).numpy()


@pytest.mark.parametrize("bs,P", [(64, 3), (64, 7), (16, 5)])
def test_partials_match_torch_per_range(bs, P):
    """Each exported partial is the attention restricted to its 16-key-rounded range (torch's
    softmax and logsumexp over an explicit mask), empty ranges give 0 / -inf, whatever BS."""
    w = small_workload([100, 37, 0], [1, 8, 1], bs=bs, seed=7)   # tokens 29-31 of seq 1 see no key of [32, 37)
    cache = written_cache(w)
    qb = w.q.view(torch.int16).numpy().view(np.uint16)
    po, pl = R.paged_attention_partials(qb, w.query_start_loc.numpy(), w.seq_lens.numpy(),
                                        w.block_tables.numpy(), cache, spec_of(w), w.softmax_scale, P)
    qsl = w.query_start_loc.tolist()
    for b, S in enumerate(w.seq_lens.tolist()):
        rows = slice(qsl[b], qsl[b + 1])
        for p, (lo, hi) in enumerate(R.partition_ranges(S, P)):
            if hi <= lo:
                assert np.all(po[rows, :, p] == 0) and np.all(np.isneginf(pl[rows, :, p]))
                continue
            o, l = _sdpa_range(w, cache, b, lo, hi)
            fin = np.isfinite(l)
            assert np.array_equal(np.isneginf(pl[rows, :, p]), ~fin)      # a token whose keys all lie later
            np.testing.assert_allclose(po[rows, :, p][fin], o[fin], rtol=0, atol=1e-12)
            np.testing.assert_allclose(pl[rows, :, p][fin], l[fin], rtol=0, atol=1e-12)
            assert np.all(po[rows, :, p][~fin] == 0)


def test_merge_edge_cases():
    po = np.random.default_rng(0).standard_normal((3, 2, 4, 5))
    pl = np.full((3, 2, 4), -np.inf)
    out, lse = R.merge_lse(po * 0, pl)
    assert np.all(out == 0) and np.all(np.isneginf(lse)) and not np.any(np.isnan(out))
    # one live partition: passes through unchanged
    pl1 = pl.copy()
    pl1[..., 2] = 1.5
    out, lse = R.merge_lse(po, pl1)
    np.testing.assert_allclose(out, po[..., 2, :], atol=1e-15)
    np.testing.assert_allclose(lse, 1.5, atol=1e-15)
    # two equal partitions: lse + ln 2, output their mean
    pl2 = np.zeros((1, 1, 2))
    po2 = np.array([[[[1.0, 2.0], [3.0, 6.0]]]])
    out, lse = R.merge_lse(po2, pl2)
    np.testing.assert_allclose(out[0, 0], [2.0, 4.0])
    np.testing.assert_allclose(lse[0, 0], math.log(2.0))


def test_padded_heads_leave_real_heads_unchanged():
    """12 real heads vs the same 12 plus 4 zero heads (vLLM PR #50371's padding check)."""
    w = small_workload([40, 9], [1, 1], hq=12, hkv=1, dk=576, dv=512, v_off=0, row=576)
    cache = written_cache(w)
    out12, lse12 = run_oracle(w, cache)
    w16 = small_workload([40, 9], [1, 1], hq=12, hkv=1, dk=576, dv=512, v_off=0, row=576)
    w16.q = torch.cat([w.q, torch.zeros(w.q.shape[0], 4, 576, dtype=torch.bfloat16)], dim=1)
    w16.num_q_heads = 16
    out16, lse16 = run_oracle(w16, cache)
    assert np.array_equal(out16[:, :12], out12) and np.array_equal(lse16[:, :12], lse12)
    # a zero query weights the visible V rows uniformly: the padded heads give their mean, not 0
    assert np.all(np.abs(out16[:, 12:]).max(axis=-1) > 0)
