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

// One step of the bit search below: candidate c = v | BIT, n = #keys >= c
// (two compares into separate scalar masks, two scalar popcounts), v = c when
// n >= Tg, and a jump to the exit when n == Tg. The exit test runs on the
// vector ALU (every lane compares the scalar n with Tg; the branch reads VCC):
// scalar issue (one scalar instruction per SIMD every four cycles) is the
// search's main limit, and this leaves six scalar and three vector
// instructions a step.
#define SPARK_SEL_STEP(BIT)                          \
    "s_or_b32 %[c], %[v], " BIT "\n\t"              \
    "v_cmp_le_u32_e64 %[m0], %[c], %[k0]\n\t"       \
    "v_cmp_le_u32_e64 %[m1], %[c], %[k1]\n\t"       \
    "s_bcnt1_i32_b64 %[x], %[m0]\n\t"               \
    "s_bcnt1_i32_b64 %[y], %[m1]\n\t"               \
    "s_add_u32 %[n], %[x], %[y]\n\t"                \
    "s_cmp_lt_u32 %[n], %[T]\n\t"                   \
    "s_cselect_b32 %[v], %[v], %[c]\n\t"            \
    "v_cmp_eq_u32 vcc, %[n], %[Tv]\n\t"             \
    "s_cbranch_vccnz 1f\n\t"

// Threshold of the Tg largest of the wave's 128 keys (two per lane; every
// lane of the wave active): v, and whether exactly Tg keys are >= v. v, n and
// the step state are wave-uniform (scalar registers); the 31 steps are
// unrolled, and the search leaves at the first count of exactly Tg. A search
// that never meets that count leaves v at 0 or at an accepted candidate, and
// more than Tg keys are >= v in both cases (0 < Tg < 128).
__device__ __forceinline__ bool search_threshold(uint32_t key0, uint32_t key1, int Tg, uint32_t& v) {
    uint32_t c, x, y, n, ex;
    uint64_t m0, m1;
    const int Tv = Tg;
    asm volatile(
        "s_mov_b32 %[v], 0\n\t"
        SPARK_SEL_STEP("0x40000000") SPARK_SEL_STEP("0x20000000") SPARK_SEL_STEP("0x10000000")
        SPARK_SEL_STEP("0x8000000") SPARK_SEL_STEP("0x4000000") SPARK_SEL_STEP("0x2000000")
        SPARK_SEL_STEP("0x1000000") SPARK_SEL_STEP("0x800000") SPARK_SEL_STEP("0x400000")
        SPARK_SEL_STEP("0x200000") SPARK_SEL_STEP("0x100000") SPARK_SEL_STEP("0x80000")
        SPARK_SEL_STEP("0x40000") SPARK_SEL_STEP("0x20000") SPARK_SEL_STEP("0x10000")
        SPARK_SEL_STEP("0x8000") SPARK_SEL_STEP("0x4000") SPARK_SEL_STEP("0x2000")
        SPARK_SEL_STEP("0x1000") SPARK_SEL_STEP("0x800") SPARK_SEL_STEP("0x400")
        SPARK_SEL_STEP("0x200") SPARK_SEL_STEP("0x100") SPARK_SEL_STEP("0x80")
        SPARK_SEL_STEP("0x40") SPARK_SEL_STEP("0x20") SPARK_SEL_STEP("0x10")
        SPARK_SEL_STEP("0x8") SPARK_SEL_STEP("0x4") SPARK_SEL_STEP("0x2")
        SPARK_SEL_STEP("0x1")
        "s_mov_b32 %[ex], 0\n\t"
        "s_branch 2f\n"
        "1:\n\t"
        "s_mov_b32 %[ex], 1\n"
        "2:"
        : [v] "=&s"(v), [c] "=&s"(c), [x] "=&s"(x), [y] "=&s"(y), [n] "=&s"(n), [ex] "=&s"(ex), [m0] "=&s"(m0),
          [m1] "=&s"(m1)
        : [k0] "v"(key0), [k1] "v"(key1), [T] "s"(Tg), [Tv] "v"(Tv)
        : "vcc", "scc");
    return ex != 0;
}

// More than Tg keys are >= v: all keys > v, then the keys equal to v in
// ascending channel order until Tg are kept.
__device__ __forceinline__ void take_ties(uint32_t key0, uint32_t key1, int Tg, uint32_t v, bool& kept0, bool& kept1) {
    const bool gt0 = key0 > v, gt1 = key1 > v;
    const int need = Tg - (__popcll(ballot(gt0)) + __popcll(ballot(gt1)));
    const uint64_t eq0 = ballot(key0 == v), eq1 = ballot(key1 == v);
    const int r0 = (int)mbcnt(eq0);
    const int r1 = __popcll(eq0) + (int)mbcnt(eq1);
    kept0 = gt0 || (key0 == v && r0 < need);
    kept1 = gt1 || (key1 == v && r1 < need);
}

// The Tg keys at or above the Tg-th largest of the wave's 128 keys, ties to
// the lower channel, as per-lane flags. (SparK-g runs it per group on keys + 1
// of the group's members and 0 elsewhere.)
__device__ __forceinline__ void select_top(uint32_t key0, uint32_t key1, int Tg, bool& kept0, bool& kept1) {
    uint32_t v;
    if (search_threshold(key0, key1, Tg, v)) {
        kept0 = key0 >= v;
        kept1 = key1 >= v;
    } else {
        take_ties(key0, key1, Tg, v, kept0, kept1);
    }
}

// The same selection as the two 64-lane masks (channels 0-63, 64-127).
__device__ __forceinline__ void select_top_masks(uint32_t key0, uint32_t key1, int Tg, uint64_t& m0, uint64_t& m1) {
    uint32_t v;
    if (search_threshold(key0, key1, Tg, v)) {
        m0 = ballot(key0 >= v);
        m1 = ballot(key1 >= v);
    } else {
        bool k0, k1;
        take_ties(key0, key1, Tg, v, k0, k1);
        m0 = ballot(k0);
        m1 = ballot(k1);
    }
}

// Lane L's bit of the wave mask m picks b (set) or a (clear): one vector
// select with the mask as its condition operand.
__device__ __forceinline__ uint32_t lane_pick(uint64_t m, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(m));
    return r;
}

// fp32 sum over the wave of each lane's x (= w_L + w_{L+64}): the pairwise
// tree that folds lanes L + 32 onto L, then L + 16, ..., L + 1. Lane L and its
// partner add the same two values, so every lane ends with the same sum.
//
// No step goes through LDS: the 32 and 16 steps are gfx950 permlane swaps,
// the others DPP moves inside each 16-lane row. After the 8 step, lanes L
// and L ^ 8 hold the same value, so the row rotation by 4 (lane (L + 4) mod
// 16) delivers lane L ^ 4's value; the last two steps are quad permutes.
// Each DPP step is written as a move with no old value, which the compiler
// folds into the add (one v_add_f32_dpp; none of these patterns reads
// outside its row, so the bound control setting never applies).
__device__ __forceinline__ float tree_sum_wave(float x) {
    x = xor32_sum(x);
    x = xor16_sum(x);
    int v = __float_as_int(x);
    x = __fadd_rn(x, __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true)));   // row_ror:8
    v = __float_as_int(x);
    x = __fadd_rn(x, __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, true)));   // row_ror:4
    v = __float_as_int(x);
    x = __fadd_rn(x, __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true)));    // quad_perm 2,3,0,1
    v = __float_as_int(x);
    x = __fadd_rn(x, __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true)));    // quad_perm 1,0,3,2
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
// SparK-g with groups of SZ = 16 or 32 channels: a key's rank in its group
// is the number of members with a larger key, so the member is kept when its
// rank is below the group's T_i. One pass over the group's keys in LDS (the
// lanes of a group read the same words) replaces a bit search per group.
// Equal keys get the same rank, so a tie that straddles T_i keeps too many;
// the group's kept count shows it, and only then is that group decided again
// by the exact bit search (ties to the lower channel).
template <int SZ>
__device__ __forceinline__ void group_ranks(const uint32_t* row, uint32_t key0, uint32_t key1, int base0, int base1,
                                            int& r0, int& r1) {
    r0 = 0;
    r1 = 0;
    const uint4* q0 = reinterpret_cast<const uint4*>(row + base0);
    const uint4* q1 = reinterpret_cast<const uint4*>(row + base1);
#pragma unroll
    for (int j = 0; j < SZ / 4; ++j) {
        const uint4 a = q0[j], b = q1[j];
        r0 += (a.x > key0) + (a.y > key0) + (a.z > key0) + (a.w > key0);
        r1 += (b.x > key1) + (b.y > key1) + (b.z > key1) + (b.w > key1);
    }
}

__device__ __forceinline__ void select_grouped_rank(uint32_t key0, uint32_t key1, int g0, int g1, int slot0,
                                                    int slot1, int T0, int T1, const GroupSpec& grp, uint32_t* row,
                                                    bool& kept0, bool& kept1) {
    row[slot0] = key0;
    row[slot1] = key1;
    wave_lds_sync();
    int r0, r1;
    if (grp.size == 32) group_ranks<32>(row, key0, key1, g0 * 32, g1 * 32, r0, r1);
    else group_ranks<16>(row, key0, key1, g0 * 16, g1 * 16, r0, r1);
    wave_lds_sync();      // every lane has read the row before the next token's keys overwrite it
    kept0 = r0 < T0;
    kept1 = r1 < T1;
    for (int i = 0; i < grp.n; ++i) {       // uniform
        const int Ti = grp.T[i];
        if (Ti <= 0 || Ti >= grp.size) continue;
        const bool in0 = g0 == i, in1 = g1 == i;
        const int n = __popcll(ballot(kept0 && in0)) + __popcll(ballot(kept1 && in1));
        if (n != Ti) {
            // members' keys + 1 (order and ties unchanged; keys are below
            // 2^31), others 0: the plain search counts members only
            bool k0, k1;
            select_top(in0 ? key0 + 1u : 0u, in1 ? key1 + 1u : 0u, Ti, k0, k1);
            if (in0) kept0 = k0;
            if (in1) kept1 = k1;
        }
    }
}

// Per-wave state of the token loop of select_pack_kernel.
struct SelectLoop {
    const uint16_t* kbh;        // this (b, kv head)'s K rows
    uint16_t* st;               // the wave's 4-row LDS stage
    uint32_t* gkeys;            // the wave's SparK-g LDS row
    int L, t_first, t_end, T;
    float A0, A1;
    double a0, a1;
    int g0, g1, slot0, slot1, T0, T1;
    bool rank_path, squares;
    float top_p;
    int32_t* tok_row;           // SparK-p: row_off + 1 of this (b, kv head)
    __amdgpu_buffer_rsrc_t mrsrc, prsrc;
    int t_begin;
};

// Accumulators of one wave: kept values (REC 0), kept counts, pruned |w|
// and |w|^2 (REC 2), channels kept (SparK-p).
struct SelectAcc {
    double sum0 = 0.0, sum1 = 0.0, pruned = 0.0, pruned2 = 0.0;
    int cnt0 = 0, cnt1 = 0, kept_tokens = 0;
};

// The token loop. REC: 0 sums of the kept values (mean-retained recovery);
// 1 counts only; 2 counts and the pruned saliency sums (squares too when
// squares is set). SEARCH (SEL 0): 0 < T < 128; otherwise every channel is
// kept or none.
template <int SEL, int REC, bool SEARCH>
__device__ __forceinline__ void select_tokens(const SelectLoop& p, const GroupSpec& grp, SelectAcc& acc) {
    constexpr uint32_t kDropped = 0x7FFFFFFFu;    // a buffer offset past every resource's end
    const int L = p.L;
    // the next 4 rows are loaded while the current 4 are searched
    uint4 xn = make_uint4(0, 0, 0, 0);
    if (p.t_first + (L >> 4) < p.t_end)
        xn = *reinterpret_cast<const uint4*>(p.kbh + (size_t)(p.t_first + (L >> 4)) * 128 + (L & 15) * 8);
    for (int t4 = p.t_first; t4 < p.t_end; t4 += 16) {
        const int n4 = min(4, p.t_end - t4);
        reinterpret_cast<uint4*>(p.st)[L] = xn;
        {
            const int tn = t4 + 16 + (L >> 4);
            xn = make_uint4(0, 0, 0, 0);
            if (tn < p.t_end) xn = *reinterpret_cast<const uint4*>(p.kbh + (size_t)tn * 128 + (L & 15) * 8);
        }
        wave_lds_sync();
        // one token: i-th row of the stage
        auto token = [&](const int i) {
            const int t = t4 + i;
            const uint16_t kb0 = p.st[i * 128 + L], kb1 = p.st[i * 128 + 64 + L];
            const float k0 = bf16_to_f32(kb0), k1 = bf16_to_f32(kb1);
            const uint32_t key0 = __float_as_uint(__fmul_rn(p.A0, __fmul_rn(k0, k0)));
            const uint32_t key1 = __float_as_uint(__fmul_rn(p.A1, __fmul_rn(k1, k1)));
            uint64_t m0, m1;
            if (SEL == 0) {
                if (SEARCH) {
                    select_top_masks(key0, key1, p.T, m0, m1);
                } else {
                    m0 = m1 = ballot(p.T >= 128);      // every channel or none
                }
            } else {
                bool kept0 = false, kept1 = false;
                if (SEL == 2) {
                    select_top_p(key0, key1, p.top_p, kept0, kept1);
                } else if (p.rank_path) {
                    select_grouped_rank(key0, key1, p.g0, p.g1, p.slot0, p.slot1, p.T0, p.T1, grp, p.gkeys, kept0,
                                        kept1);
                } else {
                    for (int g = 0; g < grp.n; ++g) {
                        const bool in0 = p.g0 == g, in1 = p.g1 == g;
                        const int Ti = grp.T[g];
                        if (Ti >= grp.size) {
                            kept0 |= in0;
                            kept1 |= in1;
                        } else if (Ti > 0) {
                            // members' keys + 1 (order and ties unchanged; keys
                            // are below 2^31), others 0: every candidate and the
                            // found threshold are >= 1, so the plain search over
                            // all 128 counts members only, with no membership
                            // masks
                            bool k0s, k1s;
                            select_top(in0 ? key0 + 1u : 0u, in1 ? key1 + 1u : 0u, Ti, k0s, k1s);
                            kept0 |= k0s;
                            kept1 |= k1s;
                        }
                    }
                }
                m0 = ballot(kept0);
                m1 = ballot(kept1);
            }
            // stores through buffer resources of this block's rows: a lane
            // that must not store gives an offset past the resource's end,
            // which the hardware drops, so no lane mask is switched
            {
                typedef uint32_t u32x4_b __attribute__((ext_vector_type(4)));
                const u32x4_b mw = {(uint32_t)m0, (uint32_t)(m0 >> 32), (uint32_t)m1, (uint32_t)(m1 >> 32)};
                __builtin_amdgcn_raw_buffer_store_b128(mw, p.mrsrc, L == 0 ? 16 * (t - p.t_begin) : (int)kDropped,
                                                       0, 0);
            }
            if (SEL == 2) {
                const int n = __popcll(m0) + __popcll(m1);
                if (L == 0) p.tok_row[t] = n;
                acc.kept_tokens += n;
            } else if (p.T > 0) {
                const int row = (t - p.t_begin) * p.T;
                const uint32_t o0 = 2u * (uint32_t)(row + (int)mbcnt(m0));
                const uint32_t o1 = 2u * (uint32_t)(row + __popcll(m0) + (int)mbcnt(m1));
                __builtin_amdgcn_raw_buffer_store_b16(kb0, p.prsrc, (int)lane_pick(m0, kDropped, o0), 0, 0);
                __builtin_amdgcn_raw_buffer_store_b16(kb1, p.prsrc, (int)lane_pick(m1, kDropped, o1), 0, 0);
            }
            acc.cnt0 += (int)lane_pick(m0, 0u, 1u);
            acc.cnt1 += (int)lane_pick(m1, 0u, 1u);
            if (REC == 0) {
                // a pruned entry adds +0, which leaves a sum that starts at +0
                // unchanged bit for bit (it is never -0)
                acc.sum0 += (double)__uint_as_float(lane_pick(m0, 0u, __float_as_uint(k0)));
                acc.sum1 += (double)__uint_as_float(lane_pick(m1, 0u, __float_as_uint(k1)));
            } else if (REC == 2) {
                const double p0 = p.a0 * (double)fabsf(k0), p1 = p.a1 * (double)fabsf(k1);
                const uint64_t b0 = __double_as_longlong(p0), b1 = __double_as_longlong(p1);
                const double w0 = __longlong_as_double((long long)(((uint64_t)lane_pick(m0, (uint32_t)(b0 >> 32), 0u) << 32) |
                                                                   lane_pick(m0, (uint32_t)b0, 0u)));
                const double w1 = __longlong_as_double((long long)(((uint64_t)lane_pick(m1, (uint32_t)(b1 >> 32), 0u) << 32) |
                                                                   lane_pick(m1, (uint32_t)b1, 0u)));
                acc.pruned += w0 + w1;
                if (p.squares) acc.pruned2 += w0 * w0 + w1 * w1;
            }
        };
        if (SEL == 0 && n4 == 4) {      // full groups of the plain select unrolled
#pragma unroll
            for (int i = 0; i < 4; ++i) token(i);
        } else {
            for (int i = 0; i < n4; ++i) token(i);
        }
        wave_lds_sync();
    }
}

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
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);     // scalar token loop
    const int L = threadIdx.x & 63;
    const int t_begin = blk * PRUNE_TOKENS_PER_BLOCK;
    const int t_end = min(S, t_begin + PRUNE_TOKENS_PER_BLOCK);

    SelectLoop p;
    p.L = L;
    p.t_begin = t_begin;
    p.t_first = t_begin + 4 * wave;        // wave w takes tokens t_begin + 4 (w + 4 i) .. + 3
    p.t_end = t_end;
    p.T = T;
    p.top_p = top_p;
    p.squares = recovery >= 4;
    // A == nullptr: unit channel energy, so the key is v^2 (V-channel pruning)
    p.A0 = A ? A[(size_t)bh * 128 + L] : 1.0f;
    p.A1 = A ? A[(size_t)bh * 128 + 64 + L] : 1.0f;
    p.a0 = sqrt((double)p.A0);
    p.a1 = sqrt((double)p.A1);
    p.g0 = GROUPED ? gid[(size_t)bh * 128 + L] : 0;
    p.g1 = GROUPED ? gid[(size_t)bh * 128 + 64 + L] : 0;
    // SparK-g with groups of 16 or 32 channels: each token's keys go to a
    // per-wave LDS row, group i's members at [i size, (i + 1) size) in
    // channel order; slot, group base and the group's kept count per lane
    __shared__ __align__(16) uint32_t gkeys[GROUPED ? 4 : 1][GROUPED ? 128 : 1];
    p.gkeys = gkeys[GROUPED ? wave : 0];
    p.rank_path = GROUPED && (grp.size == 16 || grp.size == 32);
    p.slot0 = p.slot1 = p.T0 = p.T1 = 0;
    if (p.rank_path) {
        for (int i = 0; i < grp.n; ++i) {       // uniform
            const uint64_t m0 = ballot(p.g0 == i), m1 = ballot(p.g1 == i);
            if (p.g0 == i) {
                p.slot0 = i * grp.size + (int)mbcnt(m0);
                p.T0 = grp.T[i];
            }
            if (p.g1 == i) {
                p.slot1 = i * grp.size + __popcll(m0) + (int)mbcnt(m1);
                p.T1 = grp.T[i];
            }
        }
    }

    p.kbh = k + (size_t)bh * S * 128;
    // outputs use the head stride S_out (a cache's capacity, >= S)
    uint16_t* pbh = (SEL != 2 && k_packed) ? k_packed + (size_t)bh * S_out * T : nullptr;
    uint32_t* mbh = mask + (size_t)bh * S_out * 4;
    p.st = reinterpret_cast<uint16_t*>(&stage[wave][0]);
    p.tok_row = SEL == 2 ? tok_cnt + (size_t)bh * (S + 1) : nullptr;      // row_off[bh][t + 1]
    // buffer resources over this block's mask rows and packed rows (word 3:
    // 32-bit data format, no swizzle)
    p.mrsrc = __builtin_amdgcn_make_buffer_rsrc(mbh + (size_t)t_begin * 4, (short)0, 16 * (t_end - t_begin),
                                               0x00020000);
    p.prsrc = __builtin_amdgcn_make_buffer_rsrc(pbh ? (void*)(pbh + (size_t)t_begin * T) : (void*)mbh, (short)0,
                                               pbh ? 2 * T * (t_end - t_begin) : 0, 0x00020000);

    SelectAcc acc;
    if (SEL == 0 && (T <= 0 || T >= 128)) {
        if (recovery == 0) select_tokens<SEL, 0, false>(p, grp, acc);
        else if (recovery < 3) select_tokens<SEL, 1, false>(p, grp, acc);
        else select_tokens<SEL, 2, false>(p, grp, acc);
    } else {
        if (recovery == 0) select_tokens<SEL, 0, true>(p, grp, acc);
        else if (recovery < 3) select_tokens<SEL, 1, true>(p, grp, acc);
        else select_tokens<SEL, 2, true>(p, grp, acc);
    }
    const double sum0 = acc.sum0, sum1 = acc.sum1, pruned = acc.pruned, pruned2 = acc.pruned2;
    const int cnt0 = acc.cnt0, cnt1 = acc.cnt1, kept_tokens = acc.kept_tokens;

    // fixed-order combination of the 4 waves, then one partial per block
    if (SEL == 2 && L == 0) red_tok[wave] = kept_tokens;
    red_sum[wave][L] = sum0;
    red_sum[wave][64 + L] = sum1;
    red_cnt[wave][L] = cnt0;
    red_cnt[wave][64 + L] = cnt1;
    if (recovery >= 3) {
        double pr = pruned, pr2 = pruned2;
        for (int o = 32; o > 0; o >>= 1) {
            pr += __shfl_xor(pr, o, 64);
            pr2 += __shfl_xor(pr2, o, 64);
        }
        if (L == 0) { red_pr[wave][0] = pr; red_pr[wave][1] = pr2; }
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
//
// Wave w packs tokens 16 w .. 16 w + 15 of the block; in round q lane L takes
// channels 8 (L & 15) .. + 7 of token 16 w + 4 q + (L >> 4), so each request
// reads four rows whole and all four rounds' rows and masks are requested
// before any is used. A kept channel goes to the token's offset plus the
// mask bits below it.
//
// The wave's 16 rows are consecutive, so their packed values fill one
// contiguous range [off[16 w], off[16 w + 16]) of the head's region. They
// are first placed in a per-wave LDS stage, shifted so that the stage and the
// region agree modulo 16 bytes; the range then goes out as whole 16-byte
// stores, and the (at most two) 16-byte chunks it shares with the
// neighbouring waves' ranges element by element.
__global__ void __launch_bounds__(256)
topp_pack_kernel(const uint16_t* __restrict__ k, const uint32_t* __restrict__ mask, uint16_t* __restrict__ k_packed,
                 int32_t* __restrict__ row_off, const int32_t* __restrict__ blk_base, int S, int nblk) {
    __shared__ int off[PRUNE_TOKENS_PER_BLOCK + 1];
    // per wave: 16 rows of at most 128 values, plus the alignment shift (< 8)
    __shared__ __align__(16) uint16_t stage[4][16 * 128 + 8];
    const int bh = blockIdx.y, blk = blockIdx.x;
    const int t_begin = blk * PRUNE_TOKENS_PER_BLOCK;
    const int nt = min(PRUNE_TOKENS_PER_BLOCK, S - t_begin);
    int32_t* ro = row_off + (size_t)bh * (S + 1);
    const int wave = threadIdx.x >> 6, L = threadIdx.x & 63;
    const int cb = L & 15;
    const uint16_t* kbh = k + (size_t)bh * S * 128;
    uint4 x[4], mw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = 16 * wave + 4 * q + (L >> 4);
        const int t = t_begin + min(i, nt - 1);
        mw[q] = *reinterpret_cast<const uint4*>(mask + ((size_t)bh * S + t) * 4);
        x[q] = *reinterpret_cast<const uint4*>(kbh + (size_t)t * 128 + 8 * cb);
    }
    if (threadIdx.x < 64) {
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
    uint16_t* pbh = k_packed + (size_t)bh * S * 128;
    // the wave's range: rows 16 w .. min(16 w + 16, nt) - 1 (tokens past nt
    // have no row: their offsets repeat the last one)
    const int r_lo = min(16 * wave, nt), r_hi = min(16 * wave + 16, nt);
    const int g0 = off[r_lo], g1 = off[r_hi];
    const int shift = g0 & 7;                // stage index shift + j <-> region element g0 + j
    uint16_t* stw = stage[wave];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = 16 * wave + 4 * q + (L >> 4);
        if (i >= nt) continue;
        const uint32_t words[4] = {mw[q].x, mw[q].y, mw[q].z, mw[q].w};
        const int wi = cb >> 2, sh = 8 * (cb & 3);
        int below = __popc(words[wi] & ((1u << sh) - 1u));
#pragma unroll
        for (int w = 0; w < 3; ++w) below += w < wi ? __popc(words[w]) : 0;
        const uint32_t byte = (words[wi] >> sh) & 0xFFu;
        // ranks are bounded by the row's count (the mask's popcount), so the
        // entries stay in the row's part of the range
        const int base = shift + (off[i] - g0) + below;
        const uint32_t e2[4] = {x[q].x, x[q].y, x[q].z, x[q].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if ((byte >> e) & 1u) {
                const uint16_t val = (uint16_t)((e & 1) ? (e2[e >> 1] >> 16) : (e2[e >> 1] & 0xFFFFu));
                stw[base + __popc(byte & ((1u << e) - 1u))] = val;
            }
        }
    }
    wave_lds_sync();
    // 16-byte chunks of the region from element g0 - shift: chunk c holds
    // region elements g0 - shift + 8 c .. + 7, the stage's entries 8 c .. + 7
    const int nchunk = (shift + (g1 - g0) + 7) >> 3;
    for (int c = L; c < nchunk; c += 64) {
        const int e0 = 8 * c;                                   // stage index of the chunk's first element
        const int lo = max(e0, shift), hi = min(e0 + 8, shift + (g1 - g0));
        uint16_t* dst = pbh + (g0 - shift) + e0;
        if (lo == e0 && hi == e0 + 8) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(stw + e0);
        } else {
            for (int j = lo; j < hi; ++j) dst[j - e0] = stw[j];
        }
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
        double pr = pruned, pr2 = pruned2;
        for (int o = 32; o > 0; o >>= 1) {
            pr += __shfl_xor(pr, o, 64);
            pr2 += __shfl_xor(pr2, o, 64);
        }
        if (L == 0) { red_pr[wave][0] = pr; red_pr[wave][1] = pr2; }
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
                    int S, int T, int nblk, int recovery, float f_const, int round_bf16) {
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
    if (round_bf16) {
        // to the nearest bfloat16, ties to even (the recovery of pruned V
        // entries is kept in the cache's own precision)
        uint32_t u = __float_as_uint(out);
        u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
        out = __uint_as_float(u);
    }
    r[(size_t)bh * 128 + j] = out;
    if (cnt) cnt[(size_t)bh * 128 + j] = (int32_t)c;
}

}  // namespace spark
