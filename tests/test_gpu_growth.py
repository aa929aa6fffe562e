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
