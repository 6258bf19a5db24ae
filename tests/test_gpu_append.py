"""GPU parity of attn_decode_splitkv_append: one decode step with its new token must give
exactly what attn_cache_write followed by attn_decode_splitkv gives (same cache bytes,
same outputs and log-sum-exps, bit for bit), and match the oracle.  Where the decode
kernel takes the write (power-of-two block sizes >= 16, DiffKV bf16/fp8 and the MLA row)
the new key's slot starts poisoned, so a read before the write would show (vLLM PR
#64064, "Details": V with its own stride and width; PR #50371, review thread: the
two-stage decode)."""
import math

import pytest
import torch

import paged_kv_cache_176_amd as pk
import workloads
from _gpu_util import Uploaded, compare, oracle_attention, split_last_keys

pytestmark = pytest.mark.gpu


def run_both(w, P):
    ua, ub = Uploaded(w), Uploaded(w)
    setup, (key, value, slots) = split_last_keys(w, ua)
    for u in (ua, ub):
        pk.cache_write(*setup, u.desc)
    pk.cache_write(key, value, slots, ua.desc)
    out_a, lse_a, _ = pk.decode_splitkv(ua.q, ua.desc, ua.bt, ua.seq_lens, w.softmax_scale, P)
    out_b, lse_b, _ = pk.decode_splitkv_append(ub.q, key, value, slots, ub.desc, ub.bt, ub.seq_lens,
                                               w.softmax_scale, P)
    torch.cuda.synchronize()
    assert torch.equal(ua.storage, ub.storage), "cache bytes differ from the separate write"
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b), "outputs differ from write + decode"
    return ub, out_b, lse_b


@pytest.mark.parametrize("kv,bs,scales", [("bf16", 16, "none"), ("bf16", 64, "none"), ("fp8", 16, "tensor"),
                                          ("fp8", 32, "head"), ("bf16", 8, "none"), ("fp8", 24, "tensor")])
def test_append_equals_write_then_decode(gpu_lib, kv, bs, scales):
    g = workloads.diffkv_geom(0, bs, kv_dtype=kv)
    lens = [700, 23, 0, 161, 1, 16, 17, 48]
    w = workloads.paged_workload("append", g, lens, [1] * len(lens), 32, 1 / math.sqrt(192), seed=71,
                                 scale_mode=scales)
    for P in (1, 5, 19):
        u, out, lse = run_both(w, P)
        ref, ref_lse = oracle_attention(w, u.cache_bytes())
        compare(out, ref, fp8=kv == "fp8", lse_gpu=lse, lse_ref=ref_lse, what=f"append {kv} bs={bs} P={P}")
        o = out[2].float().cpu()
        assert torch.all(o == 0) and not torch.any(torch.signbit(o))


def test_append_mla(gpu_lib):
    w = workloads.paged_workload("append_mla", workloads.mla_geom(0, 64), [3000, 65, 1, 0], [1, 1, 1, 1], 12,
                                 1 / math.sqrt(576), seed=72, std=0.1)
    for P in (1, 8, 64):
        u, out, lse = run_both(w, P)
        ref, ref_lse = oracle_attention(w, u.cache_bytes())
        compare(out, ref, lse_gpu=lse, lse_ref=ref_lse, what=f"append mla P={P}")


def test_append_partials_and_padding_slot(gpu_lib):
    """partials_only leaves the same partials as the separate calls; a sequence whose new
    token is padding (slot -1) reads its old key instead of writing one."""
    g = workloads.diffkv_geom(0, 16)
    w = workloads.paged_workload("append_pad", g, [300, 40], [1, 1], 32, 1 / math.sqrt(192), seed=73)
    ua, ub = Uploaded(w), Uploaded(w)
    setup, (key, value, slots) = split_last_keys(w, ua)
    for u in (ua, ub):
        pk.cache_write(*setup, u.desc)
    slots[1] = -1
    P = 6
    pk.cache_write(key, value, slots, ua.desc)
    _, _, ws_a = pk.decode_splitkv(ua.q, ua.desc, ua.bt, ua.seq_lens, w.softmax_scale, P, partials_only=True)
    _, _, ws_b = pk.decode_splitkv_append(ub.q, key, value, slots, ub.desc, ub.bt, ub.seq_lens, w.softmax_scale, P,
                                          partials_only=True)
    torch.cuda.synchronize()
    assert torch.equal(ua.storage, ub.storage)
    pa = pk.ops.workspace_views(ws_a, 2, 32, 128, P)
    pb = pk.ops.workspace_views(ws_b, 2, 32, 128, P)
    assert torch.equal(pa[0], pb[0]) and torch.equal(pa[1], pb[1])


@pytest.mark.parametrize("G", [24, 32])
def test_fp8_wide_rows_append(gpu_lib, G):
    """fp8 decode with more than 16 query heads per KV head runs the 32-row kernel, which
    does not take the new token's write: the call must launch the write first and give
    exactly what the separate calls give.  The LDS-streamed kernel's own limits admit these
    shapes, so the choice of who writes must follow the kernel the launch really runs."""
    g = workloads.diffkv_geom(0, 16, kv_dtype="fp8", num_kv_heads=1)
    lens = [600, 17, 0, 33]
    w = workloads.paged_workload("wide_app", g, lens, [1] * len(lens), G, 1 / math.sqrt(192), seed=94,
                                 scale_mode="tensor")
    ua, ub = Uploaded(w), Uploaded(w)
    setup, (key, value, slots) = split_last_keys(w, ua)
    for u in (ua, ub):
        pk.cache_write(*setup, u.desc)
    pk.cache_write(key, value, slots, ua.desc)
    P = 5
    o2, l2, _ = pk.decode_splitkv(ua.q, ua.desc, ua.bt, ua.seq_lens, w.softmax_scale, P)
    o1, l1, _ = pk.decode_splitkv_append(ub.q, key, value, slots, ub.desc, ub.bt, ub.seq_lens, w.softmax_scale, P)
    torch.cuda.synchronize()
    assert torch.equal(ua.storage, ub.storage), "the new token's row was not written"
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref, ref_lse = oracle_attention(w, ub.cache_bytes())
    compare(o1, ref, fp8=True, lse_gpu=l1, lse_ref=ref_lse, what=f"fp8 G {G} append")


def test_prepared_calls_replay_the_direct_calls(gpu_lib):
    """A PreparedCall (checks and marshalling done once) enqueues the same call again: its
    outputs equal the direct call's bit for bit, and a replay after the query is rewritten
    in place follows the new contents (the same storage, new values)."""
    w = workloads.paged_workload("prep", workloads.diffkv_geom(0, 16), [700, 33, 1], [1, 1, 1], 32,
                                 1 / math.sqrt(192), seed=131)
    u = Uploaded(w)
    setup, (key, value, slots) = split_last_keys(w, u)
    pk.cache_write(setup[0], setup[1], setup[2], u.desc)
    call = pk.decode_splitkv_append(u.q, key, value, slots, u.desc, u.bt, u.seq_lens, w.softmax_scale, 7,
                                    prepare=True)
    assert isinstance(call, pk.PreparedCall)
    call()
    ref_out, ref_lse, _ = pk.decode_splitkv_append(u.q, key, value, slots, u.desc, u.bt, u.seq_lens,
                                                   w.softmax_scale, 7)
    torch.cuda.synchronize()
    assert torch.equal(call.out, ref_out) and torch.equal(call.out_lse, ref_lse)
    u.q.mul_(-1)                                   # new contents, same storage
    call()
    new_out, new_lse, _ = pk.decode_splitkv(u.q, u.desc, u.bt, u.seq_lens, w.softmax_scale, 7)
    torch.cuda.synchronize()
    assert torch.equal(call.out, new_out) and torch.equal(call.out_lse, new_lse)
    assert not torch.equal(new_out, ref_out)
    # verify
    wv = workloads.paged_workload("prepv", workloads.diffkv_geom(0, 16, kv_dtype="fp8"), [500, 40], [4, 4], 32,
                                  1 / math.sqrt(192), seed=132, scale_mode="head")
    uv = Uploaded(wv)
    uv.write()
    vcall = pk.verify(uv.q, uv.qsl, uv.seq_lens, uv.bt, uv.desc, wv.softmax_scale, wv.max_query_len, 5, prepare=True)
    vcall()
    o, l, _ = pk.verify(uv.q, uv.qsl, uv.seq_lens, uv.bt, uv.desc, wv.softmax_scale, wv.max_query_len, 5)
    torch.cuda.synchronize()
    assert torch.equal(vcall.out, o) and torch.equal(vcall.out_lse, l)
