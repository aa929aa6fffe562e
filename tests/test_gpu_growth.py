"""GPU parity of decode-time cache growth through the C ABI, against the CPU
oracle: a prefill into a cache with spare capacity, then generated tokens
pruned with the prefill's channel energy and appended one at a time, each
followed by a decode step over the grown cache.

Masks and packed rows must match bit for bit; decode outputs must satisfy
|gpu - ref| <= 1e-3 + 2e-3 |ref| elementwise.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_decode_attention_amd import gen, ops
from sparse_decode_attention_amd.configs import WORKLOADS

from test_gpu_parity import assert_tol, dev_bf16, host, words_u32

pytestmark = pytest.mark.gpu


def growth_case(w, seed, lam, n_new, check_every=1, extra_cap=7, splits=0):
    S0 = w.S - n_new
    x = gen.numpy_layer(w, seed=seed, steps=n_new + 1)
    f = host(x)
    k, v = dev_bf16(x["k"]), dev_bf16(x["v"])
    cache = ops.GrowingCache(dev_bf16(x["q_win"]), k[:, :, :S0].contiguous(), v[:, :, :S0].contiguous(), w.n_kv, lam,
                             w.S + extra_cap)
    ref = oracle.prune(f["q_win"], f["k"][:, :, :S0], w.n_kv, lam)
    r_ref, _ = oracle.stats(f["k"][:, :, :S0], ref["mask"], ref["A"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cache.chan_energy.cpu().numpy(), ref["A"])
    assert_tol(cache.r.cpu().numpy(), r_ref, "r")
    packed, mask, vv = ref["packed"], ref["mask"], f["v"][:, :, :S0]
    for i in range(n_new):
        t = S0 + i
        cache.append(k[:, :, t].contiguous(), v[:, :, t].contiguous())
        packed, mask, vv = oracle.grow_cache(packed, mask, vv, f["k"][:, :, t:t + 1], f["v"][:, :, t:t + 1], ref["A"],
                                             ref["T"])
        if (i + 1) % check_every and i + 1 < n_new:
            continue
        out = cache.decode(dev_bf16(x["q_dec"][i]), splits=splits)
        torch.cuda.synchronize()
        want = oracle.decode_attn(f["q_dec"][i], packed, mask, vv, r_ref)
        assert_tol(out.cpu().numpy(), want, f"decode after {i + 1} appends")
    S = cache.S
    np.testing.assert_array_equal(words_u32(cache.mask)[:, :, :S], oracle.mask_words(mask))
    if ref["T"] > 0:
        np.testing.assert_array_equal(cache.k_packed[:, :, :S].view(torch.int16).cpu().numpy().view(np.uint16),
                                      gen.f32_to_bf16_bits(packed))
    np.testing.assert_array_equal(cache.v[:, :, :S].view(torch.int16).cpu().numpy().view(np.uint16),
                                  gen.f32_to_bf16_bits(vv))
    return cache


@pytest.mark.parametrize("lam,n_q,n_kv", [(0.5, 32, 8), (0.8, 32, 8), (0.7, 32, 8), (0.5, 16, 8), (0.6, 8, 2),
                                          (0.5, 64, 8)])
def test_growth_tiny(lam, n_q, n_kv):
    """Fast (G = 4, T in {26, 38, 64}) and generic kernels, one decode per append."""
    growth_case(WORKLOADS["tiny_s1k"].with_(S=1000, n_q=n_q, n_kv=n_kv), 100, lam, 20)


def test_growth_across_tile_and_split_boundaries():
    """S0 = 1000 grows past 1024 (a tile and a split boundary) with 2 splits."""
    growth_case(WORKLOADS["tiny_s1k"].with_(S=1090), 101, 0.5, 90, check_every=10, splits=2)


def test_prefill_cap_rows_equal_prefill():
    w = WORKLOADS["tiny_s1k"].with_(S=700)
    x = gen.numpy_layer(w, seed=102, steps=0)
    q_win, k, v = dev_bf16(x["q_win"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    cache = ops.GrowingCache(q_win, k, v, w.n_kv, 0.5, 900)
    plain = ops.prefill_prune(q_win, k, w.n_kv, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(cache.mask[:, :, :700], plain["mask"])
    assert torch.equal(cache.k_packed[:, :, :700], plain["k_packed"])
    assert torch.equal(cache.r, plain["r"]) and torch.equal(cache.chan_energy, plain["chan_energy"])
    assert (cache.mask[:, :, 700:] == 0).all()


def test_decode_cap_equals_decode_on_the_same_rows():
    w = WORKLOADS["tiny_s1k"].with_(S=1500)
    x = gen.numpy_layer(w, seed=103, steps=1)
    q_win, k, v = dev_bf16(x["q_win"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    cache = ops.GrowingCache(q_win, k, v, w.n_kv, 0.5, 2000)
    plain = ops.prefill_prune(q_win, k, w.n_kv, 0.5)
    q = dev_bf16(x["q_dec"][0])
    a = cache.decode(q)
    b = ops.decode_attn(q, plain["k_packed"], plain["mask"], v, plain["r"], 0.5)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_growth_full_size_s32k():
    """LLaMA-3.1-8B layer: prefill of 32704 tokens, then 64 generated tokens
    appended one by one up to S = 32768, decode checked every 16 steps."""
    growth_case(WORKLOADS["llama8b_s32k_l05"], 0, 0.5, 64, check_every=16)


def test_graph_replays_of_every_decode_variant_match_eager():
    """One graph holding a sampled-F decode, a K-and-V-pruned decode, a
    ragged (SparK-p) decode and four append + decode steps of a growing
    cache: every replay (with eager work and synchronisations between them)
    reproduces the eager results bit for bit."""
    w = WORKLOADS["tiny_s1k"].with_(S=1500)
    x = gen.numpy_layer(w, seed=104, steps=4)
    q_win, k, v = dev_bf16(x["q_win"]), dev_bf16(x["k"]), dev_bf16(x["v"])
    qs = [dev_bf16(x["q_dec"][s]) for s in range(4)]
    gs = ops.prefill_prune(q_win, k, w.n_kv, 0.5, recovery="gaussian")
    gk = ops.prefill_prune(q_win, k, w.n_kv, 0.5)
    gv = ops.prefill_prune_v(v, 0.5)
    gp = ops.prefill_prune_topp(q_win, k, w.n_kv, 0.95)
    S0 = 1496
    cache = ops.GrowingCache(q_win, k[:, :, :S0].contiguous(), v[:, :, :S0].contiguous(), w.n_kv, 0.5, 1500)
    k_new = [k[:, :, S0 + i].contiguous() for i in range(4)]
    v_new = [v[:, :, S0 + i].contiguous() for i in range(4)]
    outs = [torch.empty((w.B, w.n_q, 128), dtype=torch.float32, device="cuda:0") for _ in range(7)]

    def work():
        ops.decode_attn_sampled(qs[0], gs["k_packed"], gs["mask"], v, gs["chan_energy"], gs["r"], "gaussian", 99, 0.5,
                                out=outs[0])
        ops.decode_attn_kv(qs[1], gk["k_packed"], gk["mask"], gk["r"], gv["v_packed"], gv["v_mask"], gv["r_v"], 0.5,
                           0.5, out=outs[1])
        ops.decode_attn_ragged(qs[2], gp["k_packed"], gp["row_off"], gp["mask"], v, gp["r"], out=outs[2])
        cache.S = S0
        for i in range(4):
            cache.append(k_new[i], v_new[i])
            cache.decode(qs[i], out=outs[3 + i])

    work()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        cache.mask[:, :, S0:].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a_, b_) in enumerate(zip(outs, eager)):
            assert torch.equal(a_, b_), (rep, i)
        work()
        torch.cuda.synchronize()
