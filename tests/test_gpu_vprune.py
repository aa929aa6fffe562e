"""GPU parity of V-channel pruning (walkthrough section 4.4: K and V channels
pruned together) through the C ABI, against the CPU oracle.

V masks, packed V values and retained counts must match bit for bit; the V
recovery vector and every decode output must satisfy
|gpu - ref| <= 1e-3 + 2e-3 |ref| elementwise.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_decode_attention_amd import gen, ops
from sparse_decode_attention_amd.configs import WORKLOADS

from test_gpu_parity import assert_tol, check_prefill, dev_bf16, host, words_u32

pytestmark = pytest.mark.gpu


def check_prefill_v(x, lam_v):
    g = ops.prefill_prune_v(dev_bf16(x["v"]), lam_v)
    torch.cuda.synchronize()
    ref = oracle.prune_v(host(x)["v"], lam_v)
    assert g["T"] == ref["T"]
    np.testing.assert_array_equal(words_u32(g["v_mask"]), ref["words"])
    if ref["T"] > 0:
        np.testing.assert_array_equal(g["v_packed"].view(torch.int16).cpu().numpy().view(np.uint16),
                                      gen.f32_to_bf16_bits(ref["packed"]))
    np.testing.assert_array_equal(g["cnt"].cpu().numpy(), ref["cnt"])
    assert_tol(g["r_v"].cpu().numpy(), ref["r"], "r_v")
    return g, ref


def kv_case(w, seed, lam, lam_v, splits=0, steps=1):
    x = gen.numpy_layer(w, seed=seed, steps=steps)
    gk, refk, f = check_prefill(x, w.n_kv, lam)
    r_ref, _ = oracle.stats(f["k"], refk["mask"], refk["A"])
    gv, refv = check_prefill_v(x, lam_v)
    for s in range(steps):
        out = ops.decode_attn_kv(dev_bf16(x["q_dec"][s]), gk["k_packed"], gk["mask"], gk["r"], gv["v_packed"],
                                 gv["v_mask"], gv["r_v"], lam, lam_v, splits=splits)
        torch.cuda.synchronize()
        want = oracle.decode_attn_kv(f["q_dec"][s], refk["packed"], refk["mask"], r_ref, refv["packed"],
                                     refv["mask"], refv["r"])
        assert_tol(out.cpu().numpy(), want, f"K+V decode step {s}")
    return gk, gv, x


@pytest.mark.parametrize("lam_v", [0.0, 0.3, 0.5, 0.8, 1.0])
def test_prefill_v_tiny(lam_v):
    check_prefill_v(gen.numpy_layer(WORKLOADS["tiny_s1k"], seed=40, steps=0), lam_v)


@pytest.mark.parametrize("B,S,n_kv", [(2, 1, 8), (1, 63, 8), (2, 65, 4), (3, 1000, 2), (1, 513, 1)])
def test_prefill_v_ragged(B, S, n_kv):
    w = WORKLOADS["tiny_s1k"].with_(B=B, S=S, n_q=n_kv, n_kv=n_kv)
    check_prefill_v(gen.numpy_layer(w, seed=41, steps=0), 0.5)


def test_prefill_v_ties_go_to_the_lower_channel():
    """Rows of few distinct magnitudes: exact ties at the threshold."""
    rng = np.random.default_rng(42)
    v = rng.choice([0.0, 1.0, -1.0, 2.0, -2.0, 0.5], size=(1, 2, 300, 128)).astype(np.float32)
    x = {"v": gen.f32_to_bf16_bits(v)}
    for lam_v in (0.5, 0.7, 0.9):
        check_prefill_v(x, lam_v)


@pytest.mark.parametrize("lam,lam_v", [(0.5, 0.5), (0.8, 0.5), (0.5, 0.3), (0.7, 0.8), (0.0, 0.5), (0.5, 1.0)])
def test_decode_kv_tiny(lam, lam_v):
    kv_case(WORKLOADS["tiny_s1k"], 43, lam, lam_v, steps=2)


@pytest.mark.parametrize("B,S,n_q,n_kv,splits", [(1, 1, 32, 8, 0), (2, 63, 32, 8, 0), (1, 65, 8, 8, 2),
                                                 (2, 1000, 16, 8, 3), (1, 4097, 16, 2, 0), (1, 300, 8, 1, 5)])
def test_decode_kv_ragged_and_groups(B, S, n_q, n_kv, splits):
    kv_case(WORKLOADS["tiny_s1k"].with_(B=B, S=S, n_q=n_q, n_kv=n_kv), 44, 0.5, 0.5, splits=splits)


def test_decode_kv_lambda_v0_matches_dense_v_decode():
    w = WORKLOADS["tiny_s1k"].with_(S=2000)
    x = gen.numpy_layer(w, seed=45, steps=1)
    gk, _, _ = check_prefill(x, w.n_kv, 0.5)
    gv = ops.prefill_prune_v(dev_bf16(x["v"]), 0.0)
    q, v = dev_bf16(x["q_dec"][0]), dev_bf16(x["v"])
    a = ops.decode_attn_kv(q, gk["k_packed"], gk["mask"], gk["r"], gv["v_packed"], gv["v_mask"], gv["r_v"], 0.5, 0.0)
    b = ops.decode_attn(q, gk["k_packed"], gk["mask"], v, gk["r"], 0.5)
    torch.cuda.synchronize()
    assert_tol(a.cpu().numpy(), b.cpu().numpy(), "lambda_v=0 vs dense V")


def test_decode_kv_split_count_invariance():
    w = WORKLOADS["tiny_s1k"].with_(S=5000)
    x = gen.numpy_layer(w, seed=46, steps=1)
    gk, _, _ = check_prefill(x, w.n_kv, 0.5)
    gv = ops.prefill_prune_v(dev_bf16(x["v"]), 0.5)
    q = dev_bf16(x["q_dec"][0])
    outs = [ops.decode_attn_kv(q, gk["k_packed"], gk["mask"], gk["r"], gv["v_packed"], gv["v_mask"], gv["r_v"],
                               0.5, 0.5, splits=sp).cpu().numpy() for sp in (1, 2, 7, 0, 79, 79)]
    for o in outs[1:]:
        assert_tol(o, outs[0], "split invariance")
    np.testing.assert_array_equal(outs[4], outs[5])


@pytest.mark.parametrize("lam_v", [0.5, 0.8])
def test_decode_kv_full_size_s32k(lam_v):
    """The benchmarked shape (LLaMA-3.1-8B layer, S=32768, lambda=0.5) with V
    pruned too: V masks bitwise, every decode output within tolerance."""
    w = WORKLOADS["llama8b_s32k_l05"]
    kv_case(w, 0, w.lam, lam_v)
