"""GPU parity of SparK-g (walkthrough section 5.2: channel groups pruned at
their own ratios) through the C ABI, against the CPU oracle.

Channel energies, masks, packed values and counts must match bit for bit;
recovery vectors and decode outputs must satisfy
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

PAGE_RATIOS = [0.25, 0.5, 0.75, 1.0]


def check_grouped(x, n_kv, ratios, qagg="l2", recovery="mean_retained"):
    g = ops.prefill_prune_grouped(dev_bf16(x["q_win"]), dev_bf16(x["k"]), n_kv, ratios, qagg, recovery)
    torch.cuda.synchronize()
    f = host(x)
    ref = oracle.prune_grouped(f["q_win"], f["k"], n_kv, ratios, qagg)
    assert g["T"] == ref["T"]
    np.testing.assert_array_equal(g["chan_energy"].cpu().numpy(), ref["A"])
    np.testing.assert_array_equal(words_u32(g["mask"]), ref["words"])
    if ref["T"] > 0:
        np.testing.assert_array_equal(g["k_packed"].view(torch.int16).cpu().numpy().view(np.uint16),
                                      gen.f32_to_bf16_bits(ref["packed"]))
    r_ref, cnt_ref = oracle.stats(f["k"], ref["mask"], ref["A"], recovery)
    np.testing.assert_array_equal(g["cnt"].cpu().numpy(), cnt_ref)
    assert_tol(g["r"].cpu().numpy(), r_ref, f"r ({recovery})")
    return g, ref, f, r_ref


def grouped_decode_case(w, seed, ratios, splits=0, steps=1):
    x = gen.numpy_layer(w, seed=seed, steps=steps)
    g, ref, f, r_ref = check_grouped(x, w.n_kv, ratios)
    v = dev_bf16(x["v"])
    for s in range(steps):
        out = ops.decode_attn(dev_bf16(x["q_dec"][s]), g["k_packed"], g["mask"], v, g["r"], g["lam"], splits=splits)
        torch.cuda.synchronize()
        want = oracle.decode_attn(f["q_dec"][s], ref["packed"], ref["mask"], f["v"], r_ref)
        assert_tol(out.cpu().numpy(), want, f"grouped decode step {s}")


@pytest.mark.parametrize("ratios", [PAGE_RATIOS, [0.0, 0.5], [0.5], [0.1, 0.3, 0.5, 0.6, 0.7, 0.8, 0.9, 1.0],
                                    [1.0, 0.0, 0.5, 0.75]])
def test_grouped_prefill_tiny(ratios):
    w = WORKLOADS["tiny_s1k"]
    check_grouped(gen.numpy_layer(w, seed=60, steps=0), w.n_kv, ratios)


@pytest.mark.parametrize("recovery", ["mean_retained", "score_mean_pruned", "gaussian"])
@pytest.mark.parametrize("qagg", ["l2", "mean"])
def test_grouped_prefill_modes(recovery, qagg):
    w = WORKLOADS["tiny_s1k"].with_(S=700)
    check_grouped(gen.numpy_layer(w, seed=61, steps=0), w.n_kv, PAGE_RATIOS, qagg, recovery)


@pytest.mark.parametrize("B,S,n_q,n_kv", [(2, 1, 32, 8), (1, 63, 8, 8), (2, 65, 16, 8), (3, 1000, 16, 2)])
def test_grouped_prefill_ragged(B, S, n_q, n_kv):
    w = WORKLOADS["tiny_s1k"].with_(B=B, S=S, n_q=n_q, n_kv=n_kv, window=7)
    check_grouped(gen.numpy_layer(w, seed=62, steps=0), n_kv, PAGE_RATIOS)


def test_grouped_ties_in_energy_and_keys():
    """Few-valued energies and keys: ties in the group ranking and at every
    group's threshold."""
    rng = np.random.default_rng(63)
    q = rng.choice([0.0, 1.0, 2.0], size=(1, 2, 3, 128)).astype(np.float32)
    k = rng.choice([0.0, 1.0, -1.0, 2.0, 0.5], size=(1, 2, 400, 128)).astype(np.float32)
    x = {"q_win": gen.f32_to_bf16_bits(q), "k": gen.f32_to_bf16_bits(k)}
    for ratios in (PAGE_RATIOS, [0.5, 0.5], [0.3, 0.6, 0.9, 0.2, 0.5, 0.7, 0.1, 0.4]):
        check_grouped(x, 2, ratios)


@pytest.mark.parametrize("n_q,n_kv", [(32, 8), (16, 8), (8, 8), (64, 8)])
def test_grouped_decode(n_q, n_kv):
    """T = 48: the matrix-core kernel for G = 4, the generic one otherwise."""
    grouped_decode_case(WORKLOADS["tiny_s1k"].with_(S=1500, n_q=n_q, n_kv=n_kv), 64, PAGE_RATIOS, steps=2)


def test_grouped_full_size_s32k():
    """The benchmarked shape with the page's g = 4 ratios: masks bitwise,
    decode outputs within tolerance."""
    grouped_decode_case(WORKLOADS["llama8b_s32k_l05"], 0, PAGE_RATIOS)
