"""Full-size MLA parity that can tell a correct kernel from a broken one.

With Q and KV ~ N(0,1)*0.1 and scale 1/sqrt(576) the scores have std ~0.01: the softmax is
nearly uniform, every partition's lse is nearly the same and the running max never moves, so a
merge that weighted partitions equally, a broken lazy rescale, or a kernel that ignored Q would
still pass.  Here Q is scaled by 8 and needles are planted at 100,000 keys, at the split counts
the measured workloads use: each needle is aligned with one (token, head) row and scores about
ln(S) + c for c in {-1, 0, 1, 2}, so it carries a weight comparable to the whole background --
different for every head, in partitions far apart, on both sides of partition boundaries, at the
first key, at the last key of the last partition, and (verify) at positions that later tokens see
and earlier ones must not.  The bound is the strict one (max abs 1e-2 and RMSE 1e-3 against the
fp64 oracle on the same cache bytes; the needle rows have |elements| <= ~1).  The 12-head shape
and its padded 16-head run are vLLM PR #50371 ("Purpose", "Test Plan", "Test Result": an fp32
reference with max abs and cosine as the criteria)."""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import DEV, Uploaded, compare, log, oracle_attention, plant_needle

pytestmark = pytest.mark.gpu

S = 100000
OFFSETS = (-1.0, 0.0, 1.0, 2.0)


def chunk_of(P):
    return -(-(-(-S // P)) // 16) * 16          # ceil(S / P) rounded up to 16 keys


def decode_needles(P):
    """12 positions for heads 0..11 plus two repeats, around P's partition boundaries."""
    c = chunk_of(P)
    last = (P - 1) * c
    pos = [0, c - 1, c, 2 * c - 1, 2 * c, S // 2 + 5, last - 1, last, S - 50, S - 1, 5 * c - 1, 5 * c]
    extra = [(0, 3 * c + 7), (5, S - 2)]         # a second needle of the same strength for heads 0 and 5
    return [(h, p) for h, p in enumerate(pos)] + extra


def peaked_decode(B, P, seqs):
    w = workloads.mla_decode(B, S)
    w.q = (w.q.float() * 8).to(torch.bfloat16)
    for b in seqs:
        for h, j in decode_needles(P):
            plant_needle(w, b, j, b, h, math.log(S) + OFFSETS[h % 4])
    return w


@pytest.mark.parametrize("B,P", [(1, 224), (16, 16)])
def test_mla_decode_peaked_full_size(gpu_lib, B, P):
    seqs = [0] if B == 1 else [0, B // 2, B - 1]
    log(f"peaked MLA decode B{B} x {S}, P {P}: generating")
    w = peaked_decode(B, P, seqs)
    u = Uploaded(w)
    u.write()
    outs = {P: pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, P)}
    other = 16 if P != 16 else 224
    outs[other] = pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, other)
    log(f"oracle on seqs {seqs}")
    ref, ref_lse = oracle_attention(w, u.cache_bytes(), rows=seqs)
    assert float(np.abs(ref).max()) > 0.3, "the needles should dominate some heads"
    idx = torch.tensor(seqs, device=DEV)
    for p, (out, lse, _) in outs.items():
        compare(out[idx], ref, lse_gpu=lse[idx], lse_ref=ref_lse, what=f"peaked mla B{B} P{p}", strict=True)
    # the fused write-and-decode step as the bench runs it gives the same bits
    u2 = Uploaded(w)                              # context placed, the new token not yet written
    o2, l2, _ = pk.decode_splitkv_append(u2.q, u2.key, None, u2.slots, u2.desc, u2.bt, u2.seq_lens,
                                         w.softmax_scale, P)
    assert torch.equal(o2, outs[P][0]) and torch.equal(l2, outs[P][1])


def verify_needles(P, L=4):
    """(token, head, position): boundary needles for every token's heads, and needles at the
    draft positions S-L+i aligned with token i (visible to it and later tokens only) or with an
    EARLIER token that must not see it."""
    c = chunk_of(P)
    last = (P - 1) * c
    n = [(0, 0, c - 1), (0, 1, c), (1, 2, last - 1), (1, 3, last), (2, 4, 0), (3, 5, 2 * c),
         (2, 6, S // 3), (3, 7, S - L - 1)]
    n += [(i, 8 + i, S - L + i) for i in range(L)]              # token i's own position
    n += [(0, 9, S - 1), (1, 10, S - 2)]                      # hidden from tokens 0 and 1 by the mask
    # positions must be distinct: the (0, 9) / (1, 10) rows replace tokens 3 / 2's own needles
    seen, out = set(), []
    for t, h, j in reversed(n):
        if j not in seen:
            seen.add(j)
            out.append((t, h, j))
    return out[::-1]


@pytest.mark.parametrize("B,P", [(1, 224), (16, 16)])
def test_mla_verify_peaked_full_size(gpu_lib, B, P):
    L = 4
    seqs = [0] if B == 1 else [0, B // 2, B - 1]
    log(f"peaked MLA verify B{B} x {S}, {L} tokens, P {P}: generating")
    w = workloads.mla_verify(B, S, qlen=L)
    w.q = (w.q.float() * 8).to(torch.bfloat16)
    qsl = w.query_start_loc.tolist()
    for b in seqs:
        for k, (t, h, j) in enumerate(verify_needles(P, L)):
            plant_needle(w, b, j, qsl[b] + t, h, math.log(S) + OFFSETS[k % 4])
    u = Uploaded(w)
    u.write()
    out, lse, _ = pk.verify(u.q, u.qsl, u.seq_lens, u.bt, u.desc, w.softmax_scale, w.max_query_len, P)
    toks = [r for b in seqs for r in range(qsl[b], qsl[b + 1])]
    log(f"oracle on tokens {toks}")
    ref, ref_lse = oracle_attention(w, u.cache_bytes(), rows=toks)
    assert float(np.abs(ref).max()) > 0.3, "the needles should dominate some rows"
    idx = torch.tensor(toks, device=DEV)
    compare(out[idx], ref, lse_gpu=lse[idx], lse_ref=ref_lse, what=f"peaked mla verify B{B} P{P}", strict=True)
