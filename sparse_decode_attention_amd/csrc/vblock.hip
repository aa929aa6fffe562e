// V pruned in blocks of 8 consecutive channels (block reading of the
// norm-based V rule of walkthrough section 4.4): per token keep the nb blocks
// whose entries have the largest L2 norm, compared squared as an fp32 sum of
// the block's 8 squares (exact for bf16 v) added in channel order, ties to
// the lower block; pack the kept blocks in ascending block order.
//
// The block is the 16-byte unit in which the decode's P.V operand already
// loads V (lane (tau, oct) of a tile holds channels 8 oct .. 8 oct + 7 of
// rows 4i + tau), so a packed row is read with the same requests as a dense
// one, each either a kept block or the recovery of a pruned one.
#include "common.h"
#include "kernels.h"

namespace spark {

// Block: 4 waves over one 64-token tile of one (b, KV head). All 16 of a
// wave's tokens (4 rows of 4) are requested at once, lane L holding block
// L & 15 of row L >> 4: each request reads 4 rows whole. A lane ranks its
// block against the other 15 of its token (their norms through LDS), the
// ballot of "kept" holds the token's 16-bit block mask, and a kept block goes
// to slot popcount(mask below it) of the packed row.
//
// Block masks are written tile-interleaved (vblock_mask_index), the tail of
// the last tile as 0. Statistics: per lane fp64 sums of its block's 8
// channels over the kept tokens and their count, reduced over the 4 rows
// (butterfly) and the 4 waves (in wave order) into the tile's partials
// part_sum / part_cnt [BH][nblk][128], the layout of the keys' statistics.
__global__ void __launch_bounds__(256)
vblock_select_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ v_packed, uint16_t* __restrict__ bmask,
                     double* __restrict__ part_sum, int32_t* __restrict__ part_cnt, int S, int nb, int nblk,
                     int S_cap) {
    __shared__ uint32_t nsh[4][64];
    __shared__ double red_sum[4][128];
    __shared__ int red_cnt[4][16];
    const int bh = blockIdx.y, tile = blockIdx.x;
    const int wave = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int row = L >> 4, blk = L & 15;
    const int t_begin = tile * DECODE_TILE;
    const uint16_t* vbh = v + (size_t)bh * S * 128;
    uint16_t* pbh = nb > 0 ? v_packed + (size_t)bh * S_cap * nb * 8 : nullptr;
    uint16_t* mbh = bmask + (size_t)bh * vblock_mask_stride(S_cap);

    // wave w takes tokens t_begin + 4 (w + 4 i) + row, i = 0..3
    uint4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t_begin + 4 * (wave + 4 * i) + row;
        x[i] = make_uint4(0, 0, 0, 0);
        if (t < S) x[i] = *reinterpret_cast<const uint4*>(vbh + (size_t)t * 128 + blk * 8);
    }
    double sum[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) sum[c] = 0.0;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t_begin + 4 * (wave + 4 * i) + row;
        const bool valid = t < S;
        const uint32_t w[4] = {x[i].x, x[i].y, x[i].z, x[i].w};
        float f[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) f[c] = __uint_as_float((c & 1) ? (w[c >> 1] & 0xFFFF0000u) : (w[c >> 1] << 16));
        float nf = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) nf = __fadd_rn(nf, __fmul_rn(f[c], f[c]));
        // compared as unsigned bit patterns: the order of non-negative
        // floats, and a strict total order with the index tie rule whatever
        // the values, so exactly nb blocks are kept
        const uint32_t n = __float_as_uint(nf);
        nsh[wave][L] = n;
        wave_lds_sync();
        const uint4* nr = reinterpret_cast<const uint4*>(&nsh[wave][row * 16]);
        int rank = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 u = nr[q];
            const uint32_t e[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) rank += (e[k] > n || (e[k] == n && 4 * q + k < blk)) ? 1 : 0;
        }
        wave_lds_sync();     // every lane has read the norms before the next token's overwrite them
        const bool kept = valid && rank < nb;
        const uint32_t m16 = (uint32_t)(ballot(kept) >> (16 * row)) & 0xFFFFu;
        if (kept) {
            const int pos = __popc(m16 & ((1u << blk) - 1u));
            *reinterpret_cast<uint4*>(pbh + ((size_t)t * nb + pos) * 8) = x[i];
        }
        if (blk == 0) mbh[vblock_mask_index(t)] = (uint16_t)m16;
#pragma unroll
        for (int c = 0; c < 8; ++c) sum[c] += kept ? (double)f[c] : 0.0;
        cnt += kept ? 1 : 0;
    }
    // rows 0..3 of the wave: (r0 + r1) + (r2 + r3) for every lane's block
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        sum[c] += __shfl_xor(sum[c], 16, 64);
        sum[c] += __shfl_xor(sum[c], 32, 64);
    }
    cnt += __shfl_xor(cnt, 16, 64);
    cnt += __shfl_xor(cnt, 32, 64);
    if (L < 16) {
#pragma unroll
        for (int c = 0; c < 8; ++c) red_sum[wave][blk * 8 + c] = sum[c];
        red_cnt[wave][blk] = cnt;
    }
    __syncthreads();
    const int j = threadIdx.x;
    if (j < 128) {
        double s = red_sum[0][j];
        int k = red_cnt[0][j >> 3];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            s += red_sum[w][j];
            k += red_cnt[w][j >> 3];
        }
        part_sum[((size_t)bh * nblk + tile) * 128 + j] = s;
        part_cnt[((size_t)bh * nblk + tile) * 128 + j] = k;
    }
}

}  // namespace spark
