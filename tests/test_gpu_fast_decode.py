"""GPU parity of the matrix-core decode kernel's general variants through the
C ABI: every group size G in {1, 2, 4, 8}, row lengths T from 1 to 128 (odd
and even, in every row-length bucket of the kernel), and ragged SparK-p rows,
against the CPU oracle's decode (walkthrough section 3.3: pruned channels
take r, then softmax(q K^T / sqrt(D)) V).

Caches are built directly on the host: per token a random set of exactly T
kept channels, its values packed back to back in ascending channel order.
Decode outputs must satisfy |gpu - ref| <= 1e-3 + 2e-3 |ref| elementwise.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_decode_attention_amd import gen, ops

from test_gpu_parity import assert_tol, dev_bf16
from test_gpu_topp import hand_built_ragged

pytestmark = pytest.mark.gpu

D = 128


def hand_built_fixed(B, H, S, T, G, seed):
    """A fixed-T cache: mask with exactly T channels per token, packed
    [B][H][S][T], q [B][H*G][D], V dense, r random."""
    rng = np.random.default_rng(seed)
    ranks = rng.random((B, H, S, D)).argsort(-1).argsort(-1)
    mask = ranks < T
    kbits = gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D)).astype(np.float32))
    vbits = gen.f32_to_bf16_bits(rng.standard_normal((B, H, S, D)).astype(np.float32))
    qbits = gen.f32_to_bf16_bits((2.0 * rng.standard_normal((B, H * G, D))).astype(np.float32))
    r = (0.3 * rng.standard_normal((B, H, D))).astype(np.float32)
    packed_bits = kbits[mask].reshape(B, H, S, T)
    words = np.packbits(mask, axis=-1, bitorder="little").view(np.uint32)   # bit b of word w: channel 32 w + b
    dev = {"q": dev_bf16(qbits), "k_packed": dev_bf16(np.ascontiguousarray(packed_bits)),
           "mask": torch.from_numpy(words.view(np.int32).copy()).to("cuda:0"), "v": dev_bf16(vbits),
           "r": torch.from_numpy(r).to("cuda:0")}
    kf = gen.bf16_bits_to_f32(kbits)
    want = oracle.decode_attn(gen.bf16_bits_to_f32(qbits), kf[mask], mask, gen.bf16_bits_to_f32(vbits), r)
    return dev, want


def lam_of(T):
    """The pruning ratio whose kept count is exactly T (exact in fp32)."""
    lam = 1.0 - T / D
    assert ops.num_kept(D, lam) == T
    return lam


# exact-T variants: G = 4 at T = 13, 26, 51, 64, 77, 90, 102, 115 and
# G = 1, 2, 8 at T = 26, 64; every other (G, T) takes the runtime-T variant of
# its bucket (32, 64, 96, 128); odd T realigned per row in both
@pytest.mark.parametrize("T", [1, 7, 13, 26, 33, 51, 64, 77, 90, 101, 102, 115, 127, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fixed_rows_every_group_and_length(G, T):
    lam = lam_of(T)
    # one block (splits = 1) of 8 waves over 2001 tokens: several tiles per
    # wave, a partial last tile, and B * H * S * T odd for odd T, so the last
    # rows end mid-dword at the end of the packed buffer
    d, want = hand_built_fixed(1, 1, 2001, T, G, seed=1000 + 10 * G + T)
    out = ops.decode_attn(d["q"], d["k_packed"], d["mask"], d["v"], d["r"], lam, splits=1)
    torch.cuda.synchronize()
    assert_tol(out.cpu().numpy(), want, f"G={G} T={T} one block")
    # several heads and batches, the default split plan
    d, want = hand_built_fixed(2, 3, 1000, T, G, seed=2000 + 10 * G + T)
    out = ops.decode_attn(d["q"], d["k_packed"], d["mask"], d["v"], d["r"], lam)
    torch.cuda.synchronize()
    assert_tol(out.cpu().numpy(), want, f"G={G} T={T} B=2 H=3")


@pytest.mark.parametrize("G", [1, 2, 8])
@pytest.mark.parametrize("T", [1, 51])
def test_fixed_rows_tiny_caches(G, T):
    """S = 1 .. 3: rows shorter than a tile, and packed buffers barely longer
    than one lane's requests (or shorter: then the generic kernel runs)."""
    lam = lam_of(T)
    for S in (1, 2, 3, 70):
        d, want = hand_built_fixed(1, 2, S, T, G, seed=3000 + S)
        out = ops.decode_attn(d["q"], d["k_packed"], d["mask"], d["v"], d["r"], lam)
        torch.cuda.synchronize()
        assert_tol(out.cpu().numpy(), want, f"G={G} T={T} S={S}")


@pytest.mark.parametrize("G", [1, 2, 8])
@pytest.mark.parametrize("splits", [0, 3])
def test_ragged_rows_every_group(G, splits):
    """Ragged SparK-p rows for the other group sizes: one head full to its
    last element (near-end rows), one with every count 0..128, one empty,
    one mixed; S spans several tiles and a ragged tail."""
    S = 600
    rng = np.random.default_rng(90 + G)
    counts = np.stack([np.full(S, 128), rng.permutation(np.arange(S) % 129), np.zeros(S, int),
                       rng.integers(60, 120, S)])[None].astype(np.int64)
    d, want = hand_built_ragged(counts, 91 + G, n_q_per_kv=G)
    out = ops.decode_attn_ragged(d["q"], d["k_packed"], d["row_off"], d["mask"], d["v"], d["r"], splits=splits)
    torch.cuda.synchronize()
    assert_tol(out.cpu().numpy(), want, f"ragged G={G}")


@pytest.mark.parametrize("G,T", [(1, 77), (8, 90), (2, 33)])
def test_runtime_variants_repeatable_and_split_invariant(G, T):
    """Same inputs, same split count: bitwise the same output (the merge
    order is fixed); other split counts agree within tolerance."""
    lam = lam_of(T)
    d, want = hand_built_fixed(1, 2, 5000, T, G, seed=4000 + T)
    outs = [ops.decode_attn(d["q"], d["k_packed"], d["mask"], d["v"], d["r"], lam, splits=sp).cpu().numpy()
            for sp in (7, 7, 1, 0, 130)]
    np.testing.assert_array_equal(outs[0], outs[1])
    for o in outs:
        assert_tol(o, want, f"G={G} T={T} splits")


def test_more_heads_than_1024_counters():
    """B * N_kv = 1040 (b, KV head) pairs, each with its own completion
    counter, over two calls in a row (every counter back at zero after the
    first); G = 4, T = 26 (exact-T kernel) and G = 2, T = 33 (runtime T)."""
    for G, T in ((4, 26), (2, 33)):
        d, want = hand_built_fixed(130, 8, 70, T, G, seed=5000 + T)
        for _ in range(2):
            out = ops.decode_attn(d["q"], d["k_packed"], d["mask"], d["v"], d["r"], lam_of(T), splits=2)
            torch.cuda.synchronize()
            assert_tol(out.cpu().numpy(), want, f"B*N_kv=1040 G={G} T={T}")


@pytest.mark.parametrize("G,T", [(4, 90), (4, 51), (8, 64), (1, 64)])
def test_full_size_variants_s32k(G, T):
    """The bench's other pruning ratios and group sizes at their full shape
    (B = 1, 8 KV heads, S = 32768, the default split plan the bench times):
    every output against the oracle."""
    d, want = hand_built_fixed(1, 8, 32768, T, G, seed=6000 + 10 * G + T)
    out = ops.decode_attn(d["q"], d["k_packed"], d["mask"], d["v"], d["r"], lam_of(T))
    torch.cuda.synchronize()
    assert_tol(out.cpu().numpy(), want, f"S=32K G={G} T={T}")
