"""GPU parity of V pruned in 8-channel blocks (block reading of the norm-based
V rule of walkthrough section 4.4) through the C ABI, against the CPU
oracle: spark_prefill_prune_vblocks and spark_decode_attn_kvb.

Block masks (after undoing the tile interleave), packed V values and
retention counts must match bit for bit; the V recovery vector and every
decode output must satisfy |gpu - ref| <= 1e-3 + 2e-3 |ref| elementwise.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_decode_attention_amd import gen, ops
from sparse_decode_attention_amd.configs import WORKLOADS

from test_gpu_parity import assert_tol, check_prefill, dev_bf16, host

pytestmark = pytest.mark.gpu


def plain_block_masks(bmask: torch.Tensor, S: int) -> np.ndarray:
    """[B][N_kv][stride] tile-interleaved u16 masks -> [B][N_kv][S] bool [16]:
    token t sits at entry 64 (t // 64) + 16 (t % 4) + (t % 64) // 4."""
    m = bmask.cpu().numpy().view(np.uint16)
    t = np.arange(S)
    idx = 64 * (t // 64) + 16 * (t % 4) + (t % 64) // 4
    words = m[..., idx]
    return ((words[..., None] >> np.arange(16)) & 1).astype(bool)


def check_prefill_vb(x, lam_v):
    v = x["v"]
    S = v.shape[2]
    g = ops.prefill_prune_vblocks(dev_bf16(v), lam_v)
    torch.cuda.synchronize()
    ref = oracle.prune_v_blocks(gen.bf16_bits_to_f32(v), lam_v)
    assert g["nb"] == ref["nb"]
    np.testing.assert_array_equal(plain_block_masks(g["v_bmask"], S), ref["block_mask"])
    # the last tile's entries past S are 0
    stride = g["v_bmask"].shape[-1]
    t = np.arange(S, stride)
    pad = g["v_bmask"].cpu().numpy()[..., 64 * (t // 64) + 16 * (t % 4) + (t % 64) // 4]
    assert (pad == 0).all()
    if ref["nb"] > 0:
        np.testing.assert_array_equal(g["v_packed"].view(torch.int16).cpu().numpy().view(np.uint16),
                                      gen.f32_to_bf16_bits(ref["packed"]))
    np.testing.assert_array_equal(g["cnt"].cpu().numpy(), ref["cnt"])
    assert_tol(g["r_v"].cpu().numpy(), ref["r"], "r_v")
    return g, ref


def kvb_case(w, seed, lam, lam_v, splits=0, steps=1):
    x = gen.numpy_layer(w, seed=seed, steps=steps)
    gk, refk, f = check_prefill(x, w.n_kv, lam)
    r_ref, _ = oracle.stats(f["k"], refk["mask"], refk["A"])
    gv, refv = check_prefill_vb(x, lam_v)
    for s in range(steps):
        out = ops.decode_attn_kvb(dev_bf16(x["q_dec"][s]), gk["k_packed"], gk["mask"], gk["r"], gv["v_packed"],
                                  gv["v_bmask"], gv["r_v"], lam, lam_v, splits=splits)
        torch.cuda.synchronize()
        want = oracle.decode_attn_kv(f["q_dec"][s], refk["packed"], refk["mask"], r_ref, refv["packed"],
                                     refv["mask"], refv["r"])
        assert_tol(out.cpu().numpy(), want, f"K + V-block decode step {s}")
    return gk, gv, x


@pytest.mark.parametrize("lam_v", [0.0, 0.3, 0.5, 0.8, 1.0])
def test_prefill_vblocks_tiny(lam_v):
    check_prefill_vb(gen.numpy_layer(WORKLOADS["tiny_s1k"], seed=60, steps=0), lam_v)


@pytest.mark.parametrize("B,S,n_kv", [(2, 1, 8), (1, 63, 8), (2, 65, 4), (3, 1000, 2), (1, 513, 1)])
def test_prefill_vblocks_ragged(B, S, n_kv):
    w = WORKLOADS["tiny_s1k"].with_(B=B, S=S, n_q=n_kv, n_kv=n_kv)
    check_prefill_vb(gen.numpy_layer(w, seed=61, steps=0), 0.5)


def test_prefill_vblocks_ties_go_to_the_lower_block():
    """Rows of few distinct magnitudes: many blocks of equal norm."""
    rng = np.random.default_rng(62)
    v = rng.choice([0.0, 1.0, -1.0, 2.0, 0.0, 0.0], size=(1, 2, 300, 128)).astype(np.float32)
    x = {"v": gen.f32_to_bf16_bits(v)}
    for lam_v in (0.5, 0.7, 0.9):
        check_prefill_vb(x, lam_v)


def test_prefill_vblocks_summation_order():
    """Blocks whose exact squared norms tie but whose fp32 sums in channel
    order differ (2^24 + 1 + 1 rounds to 2^24; 1 + 1 + 2^24 is exact)."""
    v = np.zeros((1, 1, 64, 128), dtype=np.float32)
    v[..., 0:3] = (4096.0, 1.0, -1.0)
    v[..., 8:11] = (1.0, -1.0, 4096.0)
    g, ref = check_prefill_vb({"v": gen.f32_to_bf16_bits(v)}, 1.0 - 1.0 / 16)
    assert ref["nb"] == 1 and ref["block_mask"][0, 0, :, 1].all()


@pytest.mark.parametrize("lam,lam_v", [(0.5, 0.5), (0.8, 0.5), (0.5, 0.3), (0.7, 0.8), (0.0, 0.5), (0.5, 1.0),
                                       (0.5, 0.0), (1.0, 0.5)])
def test_decode_kvb_tiny(lam, lam_v):
    """G = 4: the exact-T block kernels (T = 64, 26), runtime-T ones (T = 38,
    128), every block count from 0 to 16, and the generic kernel (T = 0)."""
    kvb_case(WORKLOADS["tiny_s1k"], 63, lam, lam_v, steps=2)


@pytest.mark.parametrize("B,S,n_q,n_kv,splits", [(1, 1, 32, 8, 0), (2, 63, 32, 8, 0), (1, 65, 8, 8, 2),
                                                 (2, 1000, 16, 8, 3), (1, 4097, 16, 2, 0), (1, 300, 8, 1, 5),
                                                 (1, 700, 64, 8, 0)])
def test_decode_kvb_ragged_and_groups(B, S, n_q, n_kv, splits):
    """Every group size (1, 2, 4, 8), partial tiles, one-token caches and
    several split plans."""
    kvb_case(WORKLOADS["tiny_s1k"].with_(B=B, S=S, n_q=n_q, n_kv=n_kv), 64, 0.5, 0.5, splits=splits)


@pytest.mark.parametrize("lam", [0.3, 0.6, 0.8])
def test_decode_kvb_other_ratios_g8(lam):
    kvb_case(WORKLOADS["tiny_s1k"].with_(S=1500, n_q=64, n_kv=8), 65, lam, 0.5)


def test_decode_kvb_lambda_v0_matches_dense_v_decode():
    w = WORKLOADS["tiny_s1k"].with_(S=2000)
    x = gen.numpy_layer(w, seed=66, steps=1)
    gk, _, _ = check_prefill(x, w.n_kv, 0.5)
    gv = ops.prefill_prune_vblocks(dev_bf16(x["v"]), 0.0)
    q, v = dev_bf16(x["q_dec"][0]), dev_bf16(x["v"])
    a = ops.decode_attn_kvb(q, gk["k_packed"], gk["mask"], gk["r"], gv["v_packed"], gv["v_bmask"], gv["r_v"], 0.5,
                            0.0)
    b = ops.decode_attn(q, gk["k_packed"], gk["mask"], v, gk["r"], 0.5)
    torch.cuda.synchronize()
    # same kernel arithmetic on the same V values: bit for bit
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())


def test_decode_kvb_split_count_invariance():
    w = WORKLOADS["tiny_s1k"].with_(S=5000)
    x = gen.numpy_layer(w, seed=67, steps=1)
    gk, _, _ = check_prefill(x, w.n_kv, 0.5)
    gv = ops.prefill_prune_vblocks(dev_bf16(x["v"]), 0.5)
    q = dev_bf16(x["q_dec"][0])
    outs = [ops.decode_attn_kvb(q, gk["k_packed"], gk["mask"], gk["r"], gv["v_packed"], gv["v_bmask"], gv["r_v"],
                                0.5, 0.5, splits=sp).cpu().numpy() for sp in (1, 2, 7, 0, 79, 79)]
    for o in outs[1:]:
        assert_tol(o, outs[0], "split invariance")
    np.testing.assert_array_equal(outs[4], outs[5])


@pytest.mark.parametrize("lam,lam_v", [(0.5, 0.5), (0.8, 0.8)])
def test_decode_kvb_full_size_s32k(lam, lam_v):
    """The benchmarked shape (LLaMA-3.1-8B layer, S=32768) with V pruned in
    blocks: block masks bitwise, every decode output within tolerance."""
    w = WORKLOADS["llama8b_s32k_l05"]
    kvb_case(w, 0, lam, lam_v)
