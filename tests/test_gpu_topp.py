"""GPU parity of SparK-p (walkthrough section 5.2: per token the fewest
channels reaching p of its total saliency) through the C ABI, against the CPU
oracle.

Channel energies, masks, row offsets, ragged packed values and counts must
match bit for bit; recovery vectors and decode outputs must satisfy
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


def check_topp(x, n_kv, p, qagg="l2", recovery="mean_retained"):
    g = ops.prefill_prune_topp(dev_bf16(x["q_win"]), dev_bf16(x["k"]), n_kv, p, qagg, recovery)
    torch.cuda.synchronize()
    f = host(x)
    ref = oracle.prune_topp(f["q_win"], f["k"], n_kv, p, qagg)
    np.testing.assert_array_equal(g["chan_energy"].cpu().numpy(), ref["A"])
    np.testing.assert_array_equal(words_u32(g["mask"]), ref["words"])
    np.testing.assert_array_equal(g["row_off"].cpu().numpy(), ref["row_off"])
    kp = g["k_packed"].view(torch.int16).cpu().numpy().view(np.uint16)
    B, H = ref["counts"].shape[:2]
    got = np.concatenate([kp[b, h, :ref["row_off"][b, h, -1]] for b in range(B) for h in range(H)])
    np.testing.assert_array_equal(got, gen.f32_to_bf16_bits(ref["packed"]))
    r_ref, cnt_ref = oracle.stats(f["k"], ref["mask"], ref["A"], recovery)
    np.testing.assert_array_equal(g["cnt"].cpu().numpy(), cnt_ref)
    assert_tol(g["r"].cpu().numpy(), r_ref, f"r ({recovery})")
    return g, ref, f, r_ref


def topp_decode_case(w, seed, p, splits=0, steps=1):
    x = gen.numpy_layer(w, seed=seed, steps=steps)
    g, ref, f, r_ref = check_topp(x, w.n_kv, p)
    v = dev_bf16(x["v"])
    for s in range(steps):
        out = ops.decode_attn_ragged(dev_bf16(x["q_dec"][s]), g["k_packed"], g["row_off"], g["mask"], v, g["r"],
                                     splits=splits)
        torch.cuda.synchronize()
        want = oracle.decode_attn(f["q_dec"][s], ref["packed"], ref["mask"], f["v"], r_ref)
        assert_tol(out.cpu().numpy(), want, f"ragged decode step {s}")
    return g, ref


@pytest.mark.parametrize("p", [0.99, 0.9, 0.5, 1.0, 0.05])
def test_topp_prefill_tiny(p):
    w = WORKLOADS["tiny_s1k"]
    check_topp(gen.numpy_layer(w, seed=80, steps=0), w.n_kv, p)


@pytest.mark.parametrize("recovery", ["mean_retained", "score_mean_pruned", "exponential"])
@pytest.mark.parametrize("qagg", ["l2", "mean"])
def test_topp_prefill_modes(recovery, qagg):
    w = WORKLOADS["tiny_s1k"].with_(S=700)
    check_topp(gen.numpy_layer(w, seed=81, steps=0), w.n_kv, 0.95, qagg, recovery)


@pytest.mark.parametrize("B,S,n_q,n_kv", [(2, 1, 32, 8), (1, 63, 8, 8), (2, 65, 16, 8), (3, 1000, 16, 2)])
def test_topp_prefill_ragged_shapes(B, S, n_q, n_kv):
    w = WORKLOADS["tiny_s1k"].with_(B=B, S=S, n_q=n_q, n_kv=n_kv, window=7)
    check_topp(gen.numpy_layer(w, seed=82, steps=0), n_kv, 0.99)


def test_topp_exact_cases_zero_rows_and_ties():
    """Unit-like energy, few-valued keys (exact sums, ties at the threshold),
    and all-zero rows, which keep nothing."""
    rng = np.random.default_rng(83)
    q = np.ones((1, 2, 1, 128), np.float32)
    k = rng.choice([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -3.0, 4.0], size=(1, 2, 300, 128)).astype(np.float32)
    k[0, 0, :5] = 0.0
    x = {"q_win": gen.f32_to_bf16_bits(q), "k": gen.f32_to_bf16_bits(k)}
    for p in (0.5, 0.75, 0.99):
        g, ref, _, _ = check_topp(x, 2, p)
        assert (ref["counts"][0, 0, :5] == 0).all()


@pytest.mark.parametrize("n_q,n_kv,splits", [(32, 8, 0), (16, 8, 3), (8, 8, 0), (64, 8, 0), (8, 2, 7)])
def test_topp_decode(n_q, n_kv, splits):
    topp_decode_case(WORKLOADS["tiny_s1k"].with_(S=1500, n_q=n_q, n_kv=n_kv), 84, 0.99, splits=splits, steps=2)


def test_topp_decode_p1_is_dense_where_nonzero():
    """p = 1 keeps every channel whose saliency the sum cannot do without; the
    decode must match the oracle over the same cache."""
    topp_decode_case(WORKLOADS["tiny_s1k"].with_(S=777), 85, 1.0)


def test_topp_full_size_s32k():
    """The benchmarked shape with the page's p = 0.99: every mask, offset and
    packed value bitwise, decode outputs within tolerance."""
    g, ref = topp_decode_case(WORKLOADS["llama8b_s32k_l05"], 0, 0.99)
    assert 0.1 < 1 - ref["counts"].mean() / 128 < 0.9


def test_topp_decode_ignores_unwritten_capacity():
    """The packed store's capacity past each head's last row is never written:
    filled with NaN before the prefill, it must not reach the output (lanes
    with short rows read past their row; those values are replaced by 0)."""
    w = WORKLOADS["tiny_s1k"].with_(S=777)
    x = gen.numpy_layer(w, seed=86, steps=1)
    kp = torch.full((w.B, w.n_kv, w.S * 128), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    g = ops.prefill_prune_topp(dev_bf16(x["q_win"]), dev_bf16(x["k"]), w.n_kv, 0.9, out={"k_packed": kp})
    out = ops.decode_attn_ragged(dev_bf16(x["q_dec"][0]), g["k_packed"], g["row_off"], g["mask"], dev_bf16(x["v"]),
                                 g["r"])
    torch.cuda.synchronize()
    f = host(x)
    ref = oracle.prune_topp(f["q_win"], f["k"], w.n_kv, 0.9)
    r_ref, _ = oracle.stats(f["k"], ref["mask"], ref["A"])
    assert_tol(out.cpu().numpy(), oracle.decode_attn(f["q_dec"][0], ref["packed"], ref["mask"], f["v"], r_ref),
               "NaN-filled capacity")


def hand_built_ragged(counts, seed, n_q_per_kv=4):
    """A ragged cache built directly from per-token counts (0..128): random
    kept channels per token, rows packed back to back from element 0 of each
    head's region, NaN in the capacity past the last row."""
    rng = np.random.default_rng(seed)
    B, H, S = counts.shape
    D = 128
    ranks = rng.random((B, H, S, D)).argsort(-1).argsort(-1)
    mask = ranks < counts[..., None]
    kbits = gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D)).astype(np.float32))
    vbits = gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D)).astype(np.float32))
    qbits = gen.f32_to_bf16_bits(rng.standard_normal((B, H * n_q_per_kv, D)).astype(np.float32))
    r = (0.3 * rng.standard_normal((B, H, D))).astype(np.float32)
    kp = torch.full((B, H, S * D), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    for b in range(B):
        for h in range(H):
            rows = kbits[b, h][mask[b, h]]
            if rows.size:
                kp[b, h, :rows.size] = dev_bf16(rows)
    row_off = np.zeros((B, H, S + 1), np.int32)
    row_off[..., 1:] = np.cumsum(counts, axis=-1)
    words = np.packbits(mask, axis=-1, bitorder="little").view(np.uint32)   # bit b of word w: channel 32 w + b
    dev = {"q": dev_bf16(qbits), "k_packed": kp, "row_off": torch.from_numpy(row_off).to("cuda:0"),
           "mask": torch.from_numpy(words.view(np.int32).copy()).to("cuda:0"), "v": dev_bf16(vbits),
           "r": torch.from_numpy(r).to("cuda:0")}
    kf = gen.bf16_bits_to_f32(kbits)
    want = oracle.decode_attn(gen.bf16_bits_to_f32(qbits), kf[mask], mask, gen.bf16_bits_to_f32(vbits), r)
    return dev, want


@pytest.mark.parametrize("splits", [0, 3])
def test_ragged_decode_full_region_and_every_count(splits):
    """Head 0 keeps all 128 channels of every token, so its region is full to
    the last element and the rows of its final tiles take the kernel's
    near-end path; head 1 mixes every count from 0 to 128 (odd and even row
    starts); head 2 keeps nothing (scores reduce to q . r). S spans several
    tiles and a ragged tail."""
    S = 600
    rng = np.random.default_rng(87)
    counts = np.stack([np.full(S, 128), rng.permutation(np.arange(S) % 129), np.zeros(S, int),
                       rng.integers(60, 120, S)])[None].astype(np.int64)
    d, want = hand_built_ragged(counts, 88)
    out = ops.decode_attn_ragged(d["q"], d["k_packed"], d["row_off"], d["mask"], d["v"], d["r"], splits=splits)
    torch.cuda.synchronize()
    assert_tol(out.cpu().numpy(), want, "hand-built ragged cache")


def test_ragged_decode_rows_at_the_end_of_full_regions_batch2():
    """B = 2, every head full to its last element but one short row near its
    end, so the last rows start at odd and even elements within the last 65
    dwords of the allocation."""
    S = 130
    counts = np.full((2, 2, S), 128, np.int64)
    counts[0, 1, -3] = 77
    counts[1, 0, -1] = 1
    counts[1, 1, -2] = 0
    d, want = hand_built_ragged(counts, 89)
    out = ops.decode_attn_ragged(d["q"], d["k_packed"], d["row_off"], d["mask"], d["v"], d["r"])
    torch.cuda.synchronize()
    assert_tol(out.cpu().numpy(), want, "full regions, short rows at the end")
