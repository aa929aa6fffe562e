// Prefill side of SparK on gfx950: channel energy of the observation window,
// per-token exact top-T channel selection, packing of the retained keys, and
// the recovery statistics (walkthrough sections 3.1-3.3, Fig. 3 prefill half).
//
// Bit-exactness: the channel energy is an fp32 sum in a fixed order (group
// head outer, window row inner) of exact bf16 squares, and the saliency key is
// one IEEE fp32 multiply A_j * k^2. Selection compares the keys' bit patterns
// as unsigned integers (non-negative floats order like their bits), so masks
// do not depend on any floating-point reduction order.
#include "common.h"
#include "kernels.h"

namespace spark {

// ---------------------------------------------------------------- channel energy
// One block per (b, kv head), one thread per channel. The G*W window rows are
// first staged in LDS with all loads in flight, then each thread sums its
// channel sequentially (row g*W + w in increasing order).
__global__ void __launch_bounds__(256)
chan_energy_kernel(const uint16_t* __restrict__ q_win, float* __restrict__ A,
                   int N_q, int N_kv, int W, int qagg) {
    __shared__ uint4 rows[CHAN_ENERGY_ROWS * 16];       // up to CHAN_ENERGY_ROWS rows of 256 B
    const int bh = blockIdx.x;
    const int b = bh / N_kv, h = bh % N_kv;
    const int G = N_q / N_kv;
    const int R = G * W;                                // stacked rows (g outer, w inner)
    // the G heads of the group are adjacent in q_win, so their W rows are contiguous
    const uint4* src = reinterpret_cast<const uint4*>(q_win + ((size_t)b * N_q + (size_t)h * G) * W * 128);
    const int j = threadIdx.x;
    float acc = 0.f;
    for (int r0 = 0; r0 < R; r0 += CHAN_ENERGY_ROWS) {
        const int nr = min(CHAN_ENERGY_ROWS, R - r0);
        __syncthreads();
        // every load of the batch in flight before the first LDS write (no
        // conditions, which would let each load sink to its write: threads
        // past the end rewrite the last chunk with the same value)
        constexpr int PER = CHAN_ENERGY_ROWS * 16 / 256;
        uint4 tmp[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) tmp[u] = src[(size_t)r0 * 16 + min((int)threadIdx.x + u * 256, nr * 16 - 1)];
#pragma unroll
        for (int u = 0; u < PER; ++u) rows[min((int)threadIdx.x + u * 256, nr * 16 - 1)] = tmp[u];
        __syncthreads();
        if (j < 128) {
            const uint16_t* rr = reinterpret_cast<const uint16_t*>(rows);
            // rows in batches of 16: the LDS reads of a batch are all in
            // flight before its (sequential) additions
            int i = 0;
            for (; i + 16 <= nr; i += 16) {
                float x[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) x[u] = bf16_to_f32(rr[(i + u) * 128 + j]);
#pragma unroll
                for (int u = 0; u < 16; ++u) acc = (qagg == 0) ? __fadd_rn(acc, __fmul_rn(x[u], x[u])) : __fadd_rn(acc, x[u]);
            }
            for (; i < nr; ++i) {
                const float x = bf16_to_f32(rr[i * 128 + j]);
                acc = (qagg == 0) ? __fadd_rn(acc, __fmul_rn(x, x)) : __fadd_rn(acc, x);
            }
        }
    }
    if (j < 128) A[(size_t)bh * 128 + j] = (qagg == 0) ? acc : __fmul_rn(acc, acc);
}

// ---------------------------------------------------------------- select + pack
// Also serves V-channel pruning (walkthrough section 4.4): with A == nullptr
// every channel energy is 1 and the key is v^2, exact for bf16 v, which ranks
// the channels of a token by |v|.
//
// Block: 4 waves over PRUNE_TOKENS_PER_BLOCK consecutive tokens of one
// (b, kv head). Each wave takes one token at a time with lane L holding
// channels L and L + 64, so the two 64-lane ballots of "kept" are the mask
// words directly (channels 0-63, 64-127).
//
// Top-T: find the T-th largest key theta by deciding its bits from the top
// (bit 30 down; bit 31 is the sign, always 0), counting keys >= candidate
// with two ballots per step. The search stops early when exactly T keys are
// >= the candidate: those T are the answer and no tie straddles it.
// Otherwise theta is exact and the channels equal to theta are taken in
// ascending channel order until T are kept.
// The Tg keys at or above the Tg-th largest of the wave's 128 keys (two per
// lane), ties to the lower channel. (SparK-g runs it per group on keys + 1 of
// the group's members and 0 elsewhere.) v, n and the loop state are
// wave-uniform (scalar registers); each unrolled step costs two compares, two
// scalar popcounts and a scalar select, and the search leaves at the first
// count of exactly Tg.
__device__ __forceinline__ void select_top(uint32_t key0, uint32_t key1, int Tg, bool& kept0, bool& kept1) {
    uint32_t v = 0;
#pragma unroll
    for (int bit = 30; bit >= 0; --bit) {
        const uint32_t c = __builtin_amdgcn_readfirstlane(v | (1u << bit));
        const int n = __popcll(ballot(key0 >= c)) + __popcll(ballot(key1 >= c));
        v = n >= Tg ? c : v;
        if (n == Tg) break;
    }
    // whether exactly Tg keys are >= v, counted once here rather than
    // carried through every step of the search
    const bool exact = __popcll(ballot(key0 >= v)) + __popcll(ballot(key1 >= v)) == Tg;
    if (exact) {
        kept0 = key0 >= v;
        kept1 = key1 >= v;
    } else {
        const bool gt0 = key0 > v, gt1 = key1 > v;
        const int need = Tg - (__popcll(ballot(gt0)) + __popcll(ballot(gt1)));
        const uint64_t eq0 = ballot(key0 == v), eq1 = ballot(key1 == v);
        const int r0 = (int)mbcnt(eq0);
        const int r1 = __popcll(eq0) + (int)mbcnt(eq1);
        kept0 = gt0 || (key0 == v && r0 < need);
        kept1 = gt1 || (key1 == v && r1 < need);
    }
}

// fp32 sum over the wave of each lane's x (= w_L + w_{L+64}): the pairwise
// tree that folds lanes L + 32 onto L, then L + 16, ..., L + 1. Lane L and its
// partner add the same two values, so every lane ends with the same sum.
__device__ __forceinline__ float tree_sum_wave(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = __fadd_rn(x, __shfl_xor(x, m, 64));
    return x;
}

// SparK-p: with w = fl32(sqrt(key)) and target = fl32(p * total), the largest
// theta whose tree sum of w over {key >= theta} reaches the target, decided
// bit by bit from the top (the sum cannot rise as theta rises); keep
// key >= theta. An all-zero row ends with theta = 2^31 - 1 and keeps nothing.
//
// The sum depends only on the set {key >= c}. The search keeps the count of
// that set at the last accepted threshold v (whose sum reaches the target)
// and at the last rejected one (whose sum does not); a candidate whose set
// equals either of them takes its decision without a tree sum, so sums run
// only where a candidate splits the keys between the two. Once the accepted
// set holds a single key more than the rejected one, no later candidate can
// change the outcome and the search stops.
__device__ __forceinline__ void select_top_p(uint32_t key0, uint32_t key1, float p, bool& kept0, bool& kept1) {
    const float w0 = sqrtf(__uint_as_float(key0)), w1 = sqrtf(__uint_as_float(key1));
    const float target = __fmul_rn(p, tree_sum_wave(__fadd_rn(w0, w1)));
    uint32_t v = 0;
    int n_acc = 128;    // |{key >= v}|: v = 0 takes every key, and its sum (the total) reaches the target
    int n_rej = -1;     // |{key >= last rejected}|; none yet
    for (int bit = 30; bit >= 0; --bit) {
        const uint32_t c = __builtin_amdgcn_readfirstlane(v | (1u << bit));
        const int n = __popcll(ballot(key0 >= c)) + __popcll(ballot(key1 >= c));
        bool take;
        if (n == n_acc) {
            take = true;
        } else if (n == n_rej) {
            take = false;
        } else {
            const float s = tree_sum_wave(__fadd_rn(key0 >= c ? w0 : 0.0f, key1 >= c ? w1 : 0.0f));
            take = __builtin_amdgcn_readfirstlane(s >= target ? 1u : 0u) != 0;
        }
        if (take) {
            v = c;
            n_acc = n;
        } else {
            n_rej = n;
        }
        // every later candidate lies between v and the last rejected one, so
        // its set lies between theirs: with one key between them it is one of
        // the two, and the accepted set is final
        if (n_acc - n_rej <= 1) break;
    }
    kept0 = key0 >= v;
    kept1 = key1 >= v;
}

// SEL: 0 top-T; 1 SparK-g, channel c in group gid[bh][c] (0..ngroups-1), each
// group keeping its own grp.T[i] members (T is their sum); 2 SparK-p with
// threshold fraction top_p: nothing is packed here (the rows are ragged); the
// token counts go to tok_cnt[bh * (S + 1) + t] (row_off + 1: its count slots)
// and the block totals to blk_cnt[bh][blk].
template <int SEL>
__global__ void __launch_bounds__(256)
select_pack_kernel(const uint16_t* __restrict__ k, const float* __restrict__ A,
                   uint16_t* __restrict__ k_packed, uint32_t* __restrict__ mask,
                   double* __restrict__ part_sum, int32_t* __restrict__ part_cnt,
                   double* __restrict__ part_pruned,
                   int S, int T, int nblk, int recovery, const uint8_t* __restrict__ gid, GroupSpec grp,
                   float top_p, int32_t* __restrict__ tok_cnt, int32_t* __restrict__ blk_cnt, int S_out) {
    constexpr bool GROUPED = SEL == 1;
    __shared__ uint4 stage[4][64];            // 4 tokens x 256 B per wave
    __shared__ double red_sum[4][128];
    __shared__ int red_cnt[4][128];
    __shared__ double red_pr[4][2];
    __shared__ int red_tok[4];

    const int bh = blockIdx.y;
    const int blk = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int L = threadIdx.x & 63;
    const int t_begin = blk * PRUNE_TOKENS_PER_BLOCK;
    const int t_end = min(S, t_begin + PRUNE_TOKENS_PER_BLOCK);

    // A == nullptr: unit channel energy, so the key is v^2 (V-channel pruning)
    const float A0 = A ? A[(size_t)bh * 128 + L] : 1.0f;
    const float A1 = A ? A[(size_t)bh * 128 + 64 + L] : 1.0f;
    const double a0 = sqrt((double)A0), a1 = sqrt((double)A1);
    const int g0 = GROUPED ? gid[(size_t)bh * 128 + L] : 0;
    const int g1 = GROUPED ? gid[(size_t)bh * 128 + 64 + L] : 0;

    double sum0 = 0.0, sum1 = 0.0, pruned = 0.0, pruned2 = 0.0;
    int cnt0 = 0, cnt1 = 0;

    const uint16_t* kbh = k + (size_t)bh * S * 128;
    // outputs use the head stride S_out (a cache's capacity, >= S)
    uint16_t* pbh = (SEL != 2 && k_packed) ? k_packed + (size_t)bh * S_out * T : nullptr;
    int kept_tokens = 0;     // SEL 2: channels kept by this wave's tokens
    uint32_t* mbh = mask + (size_t)bh * S_out * 4;
    uint16_t* st = reinterpret_cast<uint16_t*>(&stage[wave][0]);

    // wave w takes tokens t_begin + 4*(w + 4*i) .. +3
    for (int t4 = t_begin + 4 * wave; t4 < t_end; t4 += 16) {
        const int n4 = min(4, t_end - t4);
        {   // coalesced load of up to 4 token rows (16 B per lane)
            const int tok = L >> 4;
            uint4 x = make_uint4(0, 0, 0, 0);
            if (tok < n4) x = *reinterpret_cast<const uint4*>(kbh + (size_t)(t4 + tok) * 128 + (L & 15) * 8);
            stage[wave][L] = x;
        }
        wave_lds_sync();
        for (int i = 0; i < n4; ++i) {
            const int t = t4 + i;
            const uint16_t kb0 = st[i * 128 + L], kb1 = st[i * 128 + 64 + L];
            const float k0 = bf16_to_f32(kb0), k1 = bf16_to_f32(kb1);
            const uint32_t key0 = __float_as_uint(__fmul_rn(A0, __fmul_rn(k0, k0)));
            const uint32_t key1 = __float_as_uint(__fmul_rn(A1, __fmul_rn(k1, k1)));
            bool kept0 = false, kept1 = false;
            if (SEL == 2) {
                select_top_p(key0, key1, top_p, kept0, kept1);
            } else if (!GROUPED) {
                if (T >= 128) {
                    kept0 = kept1 = true;
                } else if (T > 0) {
                    select_top(key0, key1, T, kept0, kept1);
                }
            } else {
                for (int i = 0; i < grp.n; ++i) {
                    const bool in0 = g0 == i, in1 = g1 == i;
                    const int Ti = grp.T[i];
                    if (Ti >= grp.size) {
                        kept0 |= in0;
                        kept1 |= in1;
                    } else if (Ti > 0) {
                        // members' keys + 1 (order and ties unchanged; keys are
                        // below 2^31), others 0: every candidate and the found
                        // threshold are >= 1, so the plain search over all 128
                        // counts members only, with no membership masks
                        bool k0, k1;
                        select_top(in0 ? key0 + 1u : 0u, in1 ? key1 + 1u : 0u, Ti, k0, k1);
                        kept0 |= k0;
                        kept1 |= k1;
                    }
                }
            }
            const uint64_t m0 = ballot(kept0), m1 = ballot(kept1);
            if (L == 0) {
                *reinterpret_cast<uint4*>(mbh + (size_t)t * 4) =
                    make_uint4((uint32_t)m0, (uint32_t)(m0 >> 32), (uint32_t)m1, (uint32_t)(m1 >> 32));
            }
            if (SEL == 2) {
                const int n = __popcll(m0) + __popcll(m1);
                if (L == 0) tok_cnt[(size_t)bh * (S + 1) + t] = n;    // row_off[bh][t + 1]
                kept_tokens += n;
            } else {
                if (kept0) pbh[(size_t)t * T + mbcnt(m0)] = kb0;
                if (kept1) pbh[(size_t)t * T + __popcll(m0) + mbcnt(m1)] = kb1;
            }
            if (recovery == 0) {
                if (kept0) { sum0 += (double)k0; ++cnt0; }
                if (kept1) { sum1 += (double)k1; ++cnt1; }
            } else {
                cnt0 += kept0;
                cnt1 += kept1;
                if (recovery >= 3) {
                    const double w0 = kept0 ? 0.0 : a0 * (double)fabsf(k0);
                    const double w1 = kept1 ? 0.0 : a1 * (double)fabsf(k1);
                    pruned += w0 + w1;
                    if (recovery >= 4) pruned2 += w0 * w0 + w1 * w1;
                }
            }
        }
        wave_lds_sync();
    }

    // fixed-order combination of the 4 waves, then one partial per block
    if (SEL == 2 && L == 0) red_tok[wave] = kept_tokens;
    red_sum[wave][L] = sum0;
    red_sum[wave][64 + L] = sum1;
    red_cnt[wave][L] = cnt0;
    red_cnt[wave][64 + L] = cnt1;
    if (recovery >= 3) {
        double p = pruned, p2 = pruned2;
        for (int o = 32; o > 0; o >>= 1) {
            p += __shfl_xor(p, o, 64);
            p2 += __shfl_xor(p2, o, 64);
        }
        if (L == 0) { red_pr[wave][0] = p; red_pr[wave][1] = p2; }
    }
    __syncthreads();
    if (threadIdx.x < 128) {
        const int j = threadIdx.x;
        const double s = ((red_sum[0][j] + red_sum[1][j]) + red_sum[2][j]) + red_sum[3][j];
        const int c = red_cnt[0][j] + red_cnt[1][j] + red_cnt[2][j] + red_cnt[3][j];
        part_sum[((size_t)bh * nblk + blk) * 128 + j] = s;
        part_cnt[((size_t)bh * nblk + blk) * 128 + j] = c;
        if (j < 2) part_pruned[((size_t)bh * nblk + blk) * 2 + j] =
            (recovery >= 3) ? ((red_pr[0][j] + red_pr[1][j]) + red_pr[2][j]) + red_pr[3][j] : 0.0;
        if (SEL == 2 && j == 0) blk_cnt[(size_t)bh * nblk + blk] = red_tok[0] + red_tok[1] + red_tok[2] + red_tok[3];
    }
}

template __global__ void select_pack_kernel<0>(const uint16_t*, const float*, uint16_t*, uint32_t*, double*, int32_t*,
                                               double*, int, int, int, int, const uint8_t*, GroupSpec, float, int32_t*,
                                               int32_t*, int);
template __global__ void select_pack_kernel<1>(const uint16_t*, const float*, uint16_t*, uint32_t*, double*, int32_t*,
                                               double*, int, int, int, int, const uint8_t*, GroupSpec, float, int32_t*,
                                               int32_t*, int);
template __global__ void select_pack_kernel<2>(const uint16_t*, const float*, uint16_t*, uint32_t*, double*, int32_t*,
                                               double*, int, int, int, int, const uint8_t*, GroupSpec, float, int32_t*,
                                               int32_t*, int);

// ---------------------------------------------------------------- decode-time cache growth
// One wave per (b, KV head): the new token's key is pruned with the cached
// channel energy by the prefill's rule (key fl32(A k^2), top-T, ties to the
// lower channel) and written at row `pos` of the capacity-S_cap packed
// cache and mask; its V row is copied into v at `pos`.
__global__ void __launch_bounds__(64)
append_token_kernel(const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                    const float* __restrict__ A, uint16_t* __restrict__ k_packed, uint32_t* __restrict__ mask,
                    uint16_t* __restrict__ v, int T, int pos, int S_cap) {
    const int bh = blockIdx.x, L = threadIdx.x;
    const uint16_t kb0 = k_new[(size_t)bh * 128 + L], kb1 = k_new[(size_t)bh * 128 + 64 + L];
    const float k0 = bf16_to_f32(kb0), k1 = bf16_to_f32(kb1);
    const uint32_t key0 = __float_as_uint(__fmul_rn(A[(size_t)bh * 128 + L], __fmul_rn(k0, k0)));
    const uint32_t key1 = __float_as_uint(__fmul_rn(A[(size_t)bh * 128 + 64 + L], __fmul_rn(k1, k1)));
    bool kept0 = false, kept1 = false;
    if (T >= 128) {
        kept0 = kept1 = true;
    } else if (T > 0) {
        select_top(key0, key1, T, kept0, kept1);
    }
    const uint64_t m0 = ballot(kept0), m1 = ballot(kept1);
    const size_t row = (size_t)bh * S_cap + pos;
    if (L == 0)
        *reinterpret_cast<uint4*>(mask + row * 4) =
            make_uint4((uint32_t)m0, (uint32_t)(m0 >> 32), (uint32_t)m1, (uint32_t)(m1 >> 32));
    if (kept0) k_packed[row * T + mbcnt(m0)] = kb0;
    if (kept1) k_packed[row * T + __popcll(m0) + mbcnt(m1)] = kb1;
    reinterpret_cast<uint32_t*>(v + row * 128)[L] = reinterpret_cast<const uint32_t*>(v_new + (size_t)bh * 128)[L];
}

// ---------------------------------------------------------------- SparK-p ragged packing
// One wave per (b, KV head): exclusive scan of the block totals in place
// (blk_cnt becomes each block's first element offset within the head).
__global__ void __launch_bounds__(64)
topp_scan_kernel(int32_t* __restrict__ blk_cnt, int nblk) {
    const int bh = blockIdx.x, L = threadIdx.x;
    int32_t* c = blk_cnt + (size_t)bh * nblk;
    const int per = (nblk + 63) / 64, lo = min(nblk, L * per), hi = min(nblk, lo + per);
    int local = 0;
    for (int i = lo; i < hi; ++i) local += c[i];
    int incl = local;
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (L >= o) incl += y;
    }
    int run = incl - local;
    for (int i = lo; i < hi; ++i) {
        const int x = c[i];
        c[i] = run;
        run += x;
    }
}

// Grid (nblk, B*N_kv), 256 threads: turns the block's token counts (written
// by the select kernel into row_off[t + 1]) into offsets within the head,
// row_off[t + 1] = blk_base + inclusive prefix, and packs each token's kept
// values (ascending channel) at row_off[t] of the head's region (S * 128
// elements per head).
__global__ void __launch_bounds__(256)
topp_pack_kernel(const uint16_t* __restrict__ k, const uint32_t* __restrict__ mask, uint16_t* __restrict__ k_packed,
                 int32_t* __restrict__ row_off, const int32_t* __restrict__ blk_base, int S, int nblk) {
    __shared__ int off[PRUNE_TOKENS_PER_BLOCK + 1];
    const int bh = blockIdx.y, blk = blockIdx.x;
    const int t_begin = blk * PRUNE_TOKENS_PER_BLOCK;
    const int nt = min(PRUNE_TOKENS_PER_BLOCK, S - t_begin);
    int32_t* ro = row_off + (size_t)bh * (S + 1);
    if (threadIdx.x < 64) {
        const int L = threadIdx.x;
        const int n = L < nt ? ro[t_begin + L + 1] : 0;
        int incl = n;
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o, 64);
            if (L >= o) incl += y;
        }
        const int base = blk_base[(size_t)bh * nblk + blk];
        off[L + 1] = base + incl;
        if (L == 0) off[0] = base;
    }
    __syncthreads();
    if (threadIdx.x < nt) ro[t_begin + threadIdx.x + 1] = off[threadIdx.x + 1];
    if (blk == 0 && threadIdx.x == 0) ro[0] = 0;
    const int wave = threadIdx.x >> 6, L = threadIdx.x & 63;
    const uint16_t* kbh = k + (size_t)bh * S * 128;
    uint16_t* pbh = k_packed + (size_t)bh * S * 128;
    for (int i = wave; i < nt; i += 4) {
        const int t = t_begin + i;
        const uint4 mw = *reinterpret_cast<const uint4*>(mask + ((size_t)bh * S + t) * 4);
        const uint64_t m0 = ((uint64_t)mw.y << 32) | mw.x, m1 = ((uint64_t)mw.w << 32) | mw.z;
        const bool kept0 = (m0 >> L) & 1, kept1 = (m1 >> L) & 1;
        // ranks are bounded by the row's count (the mask's popcount), so the
        // writes stay in [row_off[t], row_off[t + 1])
        if (kept0) pbh[off[i] + (int)mbcnt(m0)] = kbh[(size_t)t * 128 + L];
        if (kept1) pbh[off[i] + __popcll(m0) + (int)mbcnt(m1)] = kbh[(size_t)t * 128 + 64 + L];
    }
}

// ---------------------------------------------------------------- SparK-g channel groups
// One block per (b, KV head), one thread per channel: rank by A descending
// (ties to the lower channel), group = rank / (128 / ngroups).
__global__ void __launch_bounds__(128)
channel_groups_kernel(const float* __restrict__ A, uint8_t* __restrict__ gid, int ngroups) {
    __shared__ float a[128];
    const int bh = blockIdx.x, j = threadIdx.x;
    a[j] = A[(size_t)bh * 128 + j];
    __syncthreads();
    const float x = a[j];
    int rank = 0;
    for (int i = 0; i < 128; ++i) rank += (a[i] > x || (a[i] == x && i < j)) ? 1 : 0;
    gid[(size_t)bh * 128 + j] = (uint8_t)(rank / (128 / ngroups));
}

// ---------------------------------------------------------------- stats from a stored cache
// Same partials as select_pack_kernel, read back from (packed, mask) or, for
// the pruned-score mean, from the dense keys.
__global__ void __launch_bounds__(256)
stats_partial_kernel(const uint16_t* __restrict__ k_packed, const uint32_t* __restrict__ mask,
                     const uint16_t* __restrict__ k_dense, const float* __restrict__ A,
                     double* __restrict__ part_sum, int32_t* __restrict__ part_cnt,
                     double* __restrict__ part_pruned, int S, int T, int nblk, int recovery) {
    __shared__ double red_sum[4][128];
    __shared__ int red_cnt[4][128];
    __shared__ double red_pr[4][2];
    const int bh = blockIdx.y, blk = blockIdx.x;
    const int wave = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int t_begin = blk * PRUNE_TOKENS_PER_BLOCK;
    const int t_end = min(S, t_begin + PRUNE_TOKENS_PER_BLOCK);
    const double a0 = sqrt((double)A[(size_t)bh * 128 + L]);
    const double a1 = sqrt((double)A[(size_t)bh * 128 + 64 + L]);
    double sum0 = 0.0, sum1 = 0.0, pruned = 0.0, pruned2 = 0.0;
    int cnt0 = 0, cnt1 = 0;
    for (int t = t_begin + wave; t < t_end; t += 4) {
        const uint4 mw = *reinterpret_cast<const uint4*>(mask + ((size_t)bh * S + t) * 4);
        const uint64_t m0 = ((uint64_t)mw.y << 32) | mw.x;
        const uint64_t m1 = ((uint64_t)mw.w << 32) | mw.z;
        const bool kept0 = (m0 >> L) & 1, kept1 = (m1 >> L) & 1;
        cnt0 += kept0;
        cnt1 += kept1;
        if (recovery == 0) {
            // ranks are bounded by T so a mask with extra bits cannot read past the row
            const uint16_t* row = k_packed + ((size_t)bh * S + t) * T;
            const int rk0 = (int)mbcnt(m0), rk1 = __popcll(m0) + (int)mbcnt(m1);
            if (kept0 && rk0 < T) sum0 += (double)bf16_to_f32(row[rk0]);
            if (kept1 && rk1 < T) sum1 += (double)bf16_to_f32(row[rk1]);
        } else if (recovery >= 3) {
            const uint16_t* row = k_dense + ((size_t)bh * S + t) * 128;
            const double w0 = kept0 ? 0.0 : a0 * (double)fabsf(bf16_to_f32(row[L]));
            const double w1 = kept1 ? 0.0 : a1 * (double)fabsf(bf16_to_f32(row[64 + L]));
            pruned += w0 + w1;
            if (recovery >= 4) pruned2 += w0 * w0 + w1 * w1;
        }
    }
    red_sum[wave][L] = sum0;
    red_sum[wave][64 + L] = sum1;
    red_cnt[wave][L] = cnt0;
    red_cnt[wave][64 + L] = cnt1;
    if (recovery >= 3) {
        double p = pruned, p2 = pruned2;
        for (int o = 32; o > 0; o >>= 1) {
            p += __shfl_xor(p, o, 64);
            p2 += __shfl_xor(p2, o, 64);
        }
        if (L == 0) { red_pr[wave][0] = p; red_pr[wave][1] = p2; }
    }
    __syncthreads();
    if (threadIdx.x < 128) {
        const int j = threadIdx.x;
        part_sum[((size_t)bh * nblk + blk) * 128 + j] =
            ((red_sum[0][j] + red_sum[1][j]) + red_sum[2][j]) + red_sum[3][j];
        part_cnt[((size_t)bh * nblk + blk) * 128 + j] = red_cnt[0][j] + red_cnt[1][j] + red_cnt[2][j] + red_cnt[3][j];
        if (j < 2) part_pruned[((size_t)bh * nblk + blk) * 2 + j] =
            (recovery >= 3) ? ((red_pr[0][j] + red_pr[1][j]) + red_pr[2][j]) + red_pr[3][j] : 0.0;
    }
}

// ---------------------------------------------------------------- partials -> r
// Grid (b * N_kv, STATS_CH_BLOCKS): block y takes channels 32 y .. 32 y + 31
// of one (b, kv head), so the partials are read by that many CUs per head.
// Thread (part, jl) sums a contiguous range of the block partials of its
// channel, then the STATS_PARTS ranges are added in order, so the result is
// the same on every run.
__global__ void __launch_bounds__(STATS_THREADS)
stats_reduce_kernel(const double* __restrict__ part_sum, const int32_t* __restrict__ part_cnt,
                    const double* __restrict__ part_pruned, const float* __restrict__ A,
                    float* __restrict__ r, int32_t* __restrict__ cnt,
                    int S, int T, int nblk, int recovery, float f_const) {
    constexpr int NCH = 128 / STATS_CH_BLOCKS;
    static_assert(NCH * STATS_PARTS == STATS_THREADS, "one thread per (part, channel)");
    __shared__ double sh_s[STATS_PARTS][NCH];
    __shared__ long long sh_c[STATS_PARTS][NCH];
    __shared__ double sh_p[STATS_PARTS][2];
    __shared__ long long sh_k[STATS_THREADS / 64];
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int jl = tid % NCH, part = tid / NCH;
    const int j = blockIdx.y * NCH + jl;
    const int per = (nblk + STATS_PARTS - 1) / STATS_PARTS;
    const int lo = min(nblk, part * per), hi = min(nblk, lo + per);
    double s = 0.0, p = 0.0;
    long long c = 0;
    // batches of 16 partials: their loads are all in flight before the
    // (sequential) additions
    constexpr int NBAT = 16;
    for (int b0 = lo; b0 < hi; b0 += NBAT) {
        double xs[NBAT];
        int32_t xc[NBAT];
#pragma unroll
        for (int u = 0; u < NBAT; ++u) {
            const int blk = min(b0 + u, hi - 1);
            xs[u] = part_sum[((size_t)bh * nblk + blk) * 128 + j];
            xc[u] = part_cnt[((size_t)bh * nblk + blk) * 128 + j];
        }
#pragma unroll
        for (int u = 0; u < NBAT; ++u) {
            if (b0 + u < hi) {
                s += xs[u];
                c += xc[u];
            }
        }
    }
    if (recovery >= 3 && jl < 2) {
        constexpr int NBP = 8;
        for (int b0 = lo; b0 < hi; b0 += NBP) {
            double xp[NBP];
#pragma unroll
            for (int u = 0; u < NBP; ++u) xp[u] = part_pruned[((size_t)bh * nblk + min(b0 + u, hi - 1)) * 2 + jl];
#pragma unroll
            for (int u = 0; u < NBP; ++u)
                if (b0 + u < hi) p += xp[u];
        }
        sh_p[part][jl] = p;
    }
    sh_s[part][jl] = s;
    sh_c[part][jl] = c;
    // ragged rows (T < 0) with a pruned-saliency F: the pruned count is
    // S * 128 minus every kept entry of the head, all channels (an integer
    // sum, so its order does not matter)
    long long kept_all = (long long)S * (T < 0 ? 0 : T);
    if (T < 0 && recovery >= 3) {
        long long k = 0;
        const int32_t* pc = part_cnt + (size_t)bh * nblk * 128;
        for (size_t e = tid; e < (size_t)nblk * 128; e += STATS_THREADS) k += pc[e];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) k += __shfl_xor(k, o, 64);
        if ((tid & 63) == 0) sh_k[tid >> 6] = k;
    }
    __syncthreads();
    if (part != 0) return;
    if (T < 0 && recovery >= 3) {
        kept_all = 0;
        for (int q = 0; q < STATS_THREADS / 64; ++q) kept_all += sh_k[q];
    }
    s = 0.0;
    c = 0;
#pragma unroll 8
    for (int q = 0; q < STATS_PARTS; ++q) { s += sh_s[q][jl]; c += sh_c[q][jl]; }
    float out = 0.f;
    if (recovery == 0) {
        out = c > 0 ? (float)(s / (double)c) : 0.f;
    } else if (recovery == 2) {
        out = f_const;
    } else if (recovery >= 3) {
        double p2 = 0.0;
        p = 0.0;
#pragma unroll 8
        for (int q = 0; q < STATS_PARTS; ++q) { p += sh_p[q][0]; p2 += sh_p[q][1]; }
        const double npruned = (double)S * 128.0 - (double)kept_all;
        const double mu = npruned > 0 ? p / npruned : 0.0;
        if (recovery == 3) {
            const double a = sqrt((double)A[(size_t)bh * 128 + j]);
            out = a > 0 ? (float)(mu / a) : 0.f;
        } else {
            // sampled F: (mu, sigma) of the pruned saliency in entries 0 and 1
            const double m2 = npruned > 0 ? p2 / npruned : 0.0;
            out = j == 0 ? (float)mu : j == 1 ? (float)sqrt(fmax(m2 - mu * mu, 0.0)) : 0.f;
        }
    }
    r[(size_t)bh * 128 + j] = out;
    if (cnt) cnt[(size_t)bh * 128 + j] = (int32_t)c;
}

}  // namespace spark
