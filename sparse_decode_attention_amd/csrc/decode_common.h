// Device code shared by the decode kernels (internal header): device-scope
// partial stores and loads, the V tile loader, the sampled recovery F
// (Philox4x32-10), and the end of a decode block (wave and block merge,
// split publication, and the last block's merge of all splits).
#pragma once
#include "common.h"
#include "kernels.h"

namespace spark {

namespace {

template <int G>
struct QRow { float v[G]; };

// One channel of the decode table: q'_g for the G heads of the group, then r.
// Entries are 16-byte aligned so q' is read with vector LDS loads.
template <int G>
struct alignas(16) TabEntry {
    float q[G];
    float r;
};

// Split partials cross blocks that may run on different XCDs (separate L2s).
// They are written with device-scope (sc1) stores, which complete at the
// device coherence point without writing back the whole L2.
__device__ __forceinline__ void store_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-scope loads of values written by store_dev in other blocks (which
// may run on another XCD, behind another L2): each load is itself coherent at
// device scope, so the reader needs no L2 invalidation.
__device__ __forceinline__ float load_dev(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 load_dev4(const float* p) {
    const unsigned long long* q = reinterpret_cast<const unsigned long long*>(p);
    const unsigned long long lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                       __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
}


}  // namespace


// Byte offset, from the block's finish scratch, of its own split partial
// ((m, l) then acc, fp32): past both the block combine area and the split
// merge scratch, so it survives from the combine into the merge.
__host__ __device__ inline uint32_t finish_own_offset(int G, int NT, int nsplit) {
    const uint32_t combine = (uint32_t)(NT / 64) * (2u * G + (uint32_t)G * 128u) * 4u;
    const uint32_t merge = ((((uint32_t)nsplit * 3u * G + G + 3u) & ~3u) * 4u) + (uint32_t)NT * 16u;
    const uint32_t m = combine > merge ? combine : merge;
    return (m + 15u) & ~15u;
}
__host__ __device__ inline uint32_t finish_scratch_bytes(int G, int NT, int nsplit) {
    return finish_own_offset(G, NT, nsplit) + (2u * G + (uint32_t)G * 128u) * 4u;
}

// Merge the (m, l, acc) partials of all splits of one (b, KV head) and write
// out = acc / l. Runs in the block that took the last ticket, once every
// other split has published its partial with device-scope stores; those are
// read with device-scope loads, the merging block's own partial (split `own`)
// from LDS. All loads are issued in batches; every reduction has a fixed
// order, so the output does not depend on which block merges.
template <int G, int NT>
__device__ void merge_splits(const DecodeArgs& a, int bh, int b, int h, float* lds, int own,
                             const float* own_ml, const float* own_acc) {
    constexpr int NQ = G * 32;                       // float4 per split partial
    constexpr int NPH = NT / NQ;                     // threads per float4 column
    constexpr int NW = NT / 64;
    constexpr int BATCH = 8;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, L = tid & 63;
    const int ns = a.nsplit;
    float* sml = lds;                                // [ns][2][G]
    float* sf = sml + ns * 2 * G;                    // [ns][G] scale of each split
    float* sL = sf + ns * G;                         // [G] total l
    float4* sred = reinterpret_cast<float4*>(lds + ((ns * 3 * G + G + 3) & ~3));  // [NPH][NQ]
    // partials are read with device-scope loads (no acquire fence, which
    // would invalidate this XCD's L2 under the blocks still streaming)
    const float* ml_bh = a.part_ml + (size_t)bh * ns * 2 * G;
    // the first batch of acc partials is requested together with m and l
    const int q = tid % NQ, ph = tid / NQ;
    const int g = q / 32;
    const float* acc_bh = a.part_acc + (size_t)bh * ns * G * 128;
    float4 v0[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) {
        const int sp = ph + k * NPH;
        v0[k] = sp == own ? reinterpret_cast<const float4*>(own_acc)[q]
              : sp < ns   ? load_dev4(acc_bh + ((size_t)sp * NQ + q) * 4)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int i = tid; i < ns * 2 * G; i += NT)
        sml[i] = (i / (2 * G) == own) ? own_ml[i % (2 * G)] : load_dev(ml_bh + i);
    __syncthreads();
    // per head: M = max over splits, then the split scales and L = sum l * scale
    for (int hd = wave; hd < G; hd += NW) {
        float mx = -INFINITY;
        for (int sp = L; sp < ns; sp += 64) mx = fmaxf(mx, sml[sp * 2 * G + hd]);
        const float M = wave_max_dpp(mx);
        float ls = 0.f;
        for (int sp = L; sp < ns; sp += 64) {
            const float m = sml[sp * 2 * G + hd];
            const float f = (m == -INFINITY) ? 0.f : exp2f(m - M);
            sf[sp * G + hd] = f;
            ls += sml[sp * 2 * G + G + hd] * f;
        }
        ls = wave_sum_dpp(ls);
        if (L == 0) sL[hd] = ls;
    }
    __syncthreads();
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp0 = ph; sp0 < ns; sp0 += NPH * BATCH) {
        float4 v[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int sp = sp0 + k * NPH;
            if (sp0 == ph) v[k] = v0[k];
            else v[k] = sp == own ? reinterpret_cast<const float4*>(own_acc)[q]
                      : sp < ns   ? load_dev4(acc_bh + ((size_t)sp * NQ + q) * 4)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int sp = sp0 + k * NPH;
            const float f = sp < ns ? sf[sp * G + g] : 0.f;
            x.x += v[k].x * f; x.y += v[k].y * f; x.z += v[k].z * f; x.w += v[k].w * f;
        }
    }
    sred[ph * NQ + q] = x;
    __syncthreads();
    if (ph == 0) {
        float4 t = sred[q];
#pragma unroll
        for (int p = 1; p < NPH; ++p) {
            const float4 u = sred[p * NQ + q];
            t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
        }
        const float inv = 1.0f / sL[g];
        float4* o = reinterpret_cast<float4*>(a.out + ((size_t)b * a.N_q + (size_t)h * G) * 128);
        o[q] = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
    }
}

// V rows of one tile for the P.V layout: lane (tau, oct) takes rows 4i + tau,
// d in [8 oct, 8 oct + 8). Rows past the end of a partial tile re-read the
// last valid row; their p is 0.
//
// The requests are nontemporal (`global_load_dwordx4 … nt`): each one of a
// wave reads four whole 256-byte rows, so no line is wanted again, and
// streaming V past the L2 this way measured faster at every shape (S = 32K:
// 27.9 -> 26.9 us at lambda 0.5; S = 128K: 84.8 -> 74.6 us). (The packed K
// rows are not: a lane reads its row in several requests, and each of those
// would fetch the row's lines again.)
__device__ __forceinline__ void load_v_tile(const uint16_t* vbh, int t0, int nt, int tau, int oct, uint4 (&vr)[16]) {
    typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
    // 32-bit byte offsets from the head's V slab (fewer than 2^24 rows of
    // 256 B, checked on the host), so each request is a scalar base plus one
    // vector offset
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(vbh);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t row = (uint32_t)(t0 + min(4 * i + tau, nt - 1));
        const u32x4_nt x =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(vb + (row * 256u + (uint32_t)oct * 16u)));
        vr[i] = make_uint4(x.x, x.y, x.z, x.w);
    }
}

// ---- V pruned in 8-channel blocks. The 8 channels a lane (tau, oct) holds
// in the P.V layout are one block, so a pruned V cache is read with the same
// 16-byte requests as a dense one: the block from its slot in the token's
// packed row when kept, else the block's recovery values.

// The tile's block masks for rows 4i + tau (i = 0..15): entries 16 tau ..
// 16 tau + 15 of the tile's 64 interleaved masks, 32 contiguous bytes (the 16
// lanes of one tau read the same two requests). t0 is rounded down to its
// tile, so that a wave without a tile (t0 clamped to S - 1) reads in bounds.
__device__ __forceinline__ void load_vblock_masks(const uint16_t* vmh, int t0, int tau, uint4 (&vm)[2]) {
    const uint4* p = reinterpret_cast<const uint4*>(vmh + (t0 & ~(DECODE_TILE - 1)) + 16 * tau);
    vm[0] = p[0];
    vm[1] = p[1];
}

// This lane's 8 recovery values (channels 8 oct .. 8 oct + 7) as bf16 bits,
// rounded to nearest even (the prefill writes them already rounded to bf16,
// which this leaves unchanged). Taken as the two fp32 quads loaded, so that
// the loads can be issued early and converted where first needed.
__device__ __forceinline__ uint4 vblock_recovery(const float4& lo, const float4& hi) {
    const float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t u = __float_as_uint(f[e]);
        h[e] = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    }
    return make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
}

// V rows of one tile from a block-pruned cache, in load_v_tile's layout: row
// 4i + tau takes its kept block oct from slot popcount(mask below oct) of the
// packed row (nb blocks of 16 bytes); bit i of the returned mask says whether
// it was kept. A lane whose block is pruned (or whose row lies past the
// tile's end) requests slot 0 of its row, a line the row's kept blocks bring
// in anyway, so that no request is conditional; vblock_fill later puts the
// recovery block in its place. The choice is made there, where P.V needs
// the values, and not here: a select right after the requests would wait
// for them before the scores. With nb = 0 there is nothing to read. Slots
// are clamped to the row, so a mask with more than nb bits set reads wrong
// values but stays in bounds. Row offsets are 32-bit (heads of fewer than
// 2^24 tokens of at most 256 B).
__device__ __forceinline__ uint32_t load_v_tile_blocks(const uint16_t* vpbh, const uint4 (&vm)[2], int nb, int t0,
                                                       int nt, int tau, int oct, uint4 (&vr)[16]) {
    typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
    if (nb == 0) return 0u;
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(vpbh);
    const uint32_t below = (1u << oct) - 1u;
    const uint32_t row_bytes = 16u * (uint32_t)nb;
    uint32_t kbits = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint4& q = vm[i >> 3];
        const int d = (i >> 1) & 3;
        const uint32_t w = d == 0 ? q.x : d == 1 ? q.y : d == 2 ? q.z : q.w;
        const uint32_t m = (i & 1) ? (w >> 16) : (w & 0xFFFFu);
        const bool kept = 4 * i + tau < nt && ((m >> oct) & 1u) != 0u;
        const uint32_t row = (uint32_t)(t0 + min(4 * i + tau, nt - 1));
        const uint32_t slot = kept ? min((uint32_t)__popc(m & below), (uint32_t)nb - 1u) : 0u;
        const u32x4_nt x =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(vb + (row * row_bytes + 16u * slot)));
        vr[i] = make_uint4(x.x, x.y, x.z, x.w);
        kbits |= kept ? (1u << i) : 0u;
    }
    return kbits;
}

// The recovery block in every slot of vr that load_v_tile_blocks did not
// fill with a kept block.
__device__ __forceinline__ void vblock_fill(uint4 (&vr)[16], uint32_t kbits, const uint4& rvo) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (((kbits >> i) & 1u) == 0u) vr[i] = rvo;
}

// ---- sampled recovery F (walkthrough section 3.3, F table, Gaussian and
// Exponential rows): every pruned (t, j) draws its own sample.
//
// Philox4x32 with 10 rounds, from its published definition (Salmon, Moraes,
// Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011): a
// round takes the two 32 x 32 -> 64-bit products of words 0 and 2 with the
// multipliers and xors their high halves into words 1 and 3 with the round
// key; the key advances by the two Weyl constants between rounds. Each
// product is one 64-bit multiply-add on the vector ALU.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

// a ^ b ^ c in one v_bitop3_b32 (truth table 0x96: the parity of the three
// input bits, the same for any operand order).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// The first round is written with plain xors so that the compiler can fold
// its wave-uniform counter words (channel group, head) into scalar code.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int rnd = 0; rnd < 10; ++rnd) {
        if (rnd) { k0 += kPhiloxW0; k1 += kPhiloxW1; }
        const uint64_t p0 = (uint64_t)kPhiloxM0 * c.x;
        const uint64_t p1 = (uint64_t)kPhiloxM1 * c.z;
        const uint32_t h1 = (uint32_t)(p1 >> 32), h0 = (uint32_t)(p0 >> 32);
        c = rnd == 0 ? make_uint4(h1 ^ c.y ^ k0, (uint32_t)p1, h0 ^ c.w ^ k1, (uint32_t)p0)
                     : make_uint4(xor3(h1, c.y, k0), (uint32_t)p1, xor3(h0, c.w, k1), (uint32_t)p0);
    }
    return c;
}

// u = (x + 1/2) 2^-32 in [2^-33, 1], rounded to fp32 (never denormal).
__device__ __forceinline__ float unit_of(uint32_t x) { return fmaf((float)x, 0x1p-32f, 0x1p-33f); }

// Zero-mean noise of one Philox block for channels 4 jg + 0..3, from the
// hardware log2, square root, sine and cosine (the last two take their
// argument in turns, so 2 pi u needs no multiply); u is a normal number, so
// no denormal rescaling is needed. Gaussian: Box-Muller on (u0, u1) and
// (u2, u3), z_even = R cos(2 pi u_odd), z_odd = R sin(2 pi u_odd),
// R = sqrt(-2 ln u_even). Exponential: -ln u has mean 1, so the noise is
// -ln u - 1 (the sample is mu times -ln u).
template <bool GAUSS>
__device__ __forceinline__ void sample_noise4(uint4 x, float (&n)[4]) {
    constexpr float kLn2 = 0.693147180559945309f;
    const float u[4] = {unit_of(x.x), unit_of(x.y), unit_of(x.z), unit_of(x.w)};
    if (GAUSS) {
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            const float R = __builtin_amdgcn_sqrtf(-2.0f * kLn2 * __builtin_amdgcn_logf(u[e]));
            n[e] = R * __builtin_amdgcn_cosf(u[e + 1]);
            n[e + 1] = R * __builtin_amdgcn_sinf(u[e + 1]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) n[e] = fmaf(-__builtin_amdgcn_logf(u[e]), kLn2, -1.0f);
    }
}

// Sample term of the scores of one tile: with the table's r_j = mu / a_j
// (the sample mean back-solved) already in the scores, every pruned channel
// j of the lane's token adds (q'_g,j ns_j) n_tj, ns_j the noise scale of the
// back-solved sample. The counter of token t and channel group jg is
// (t, jg, b * N_kv + h, 0). The four q' ns rows of a group are read (LDS
// broadcast) before its Philox block, so they arrive during it; a kept
// channel's noise is cleared with the sign-extended mask bit; groups that
// every lane of the wave keeps are skipped.
template <int G, bool GAUSS>
__device__ __forceinline__ void sampled_scores(const DecodeArgs& a, const float* qn, uint4 mw, int bh,
                                               int t0, int nt, int L, float (&s)[G]) {
    const uint32_t tok = (uint32_t)(t0 + L);
    const bool live = L < nt;
    const uint32_t words[4] = {mw.x, mw.y, mw.z, mw.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t pr = live ? ~words[w] : 0u;
        for (int jj = 0; jj < 8; ++jj) {
            if (ballot(((pr >> (4 * jj)) & 15u) != 0) == 0) continue;
            const int jg = 8 * w + jj;
            QRow<G> row[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) row[i] = reinterpret_cast<const QRow<G>*>(qn)[4 * jg + i];
            const uint4 x = philox4x32_10(make_uint4(tok, (uint32_t)jg, (uint32_t)bh, 0u), a.seed_lo, a.seed_hi);
            float n[4];
            sample_noise4<GAUSS>(x, n);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t keep_bits = (uint32_t)__builtin_amdgcn_sbfe((int)pr, 4 * jj + i, 1);
                const float xn = __uint_as_float(__float_as_uint(n[i]) & keep_bits);
#pragma unroll
                for (int g = 0; g < G; ++g) s[g] = fmaf(row[i].v[g], xn, s[g]);
            }
        }
    }
}

// End of a decode block: reduce each wave's (m, l, acc) over its token phases
// and lanes, merge the waves in LDS, publish the block's split partial, and,
// in the last block of the (b, KV head) to finish, merge all splits.
//
// Two accumulator layouts: the VALU one (MF false), where lane (tau, oct)
// holds acc[g][e] for d = 8 oct + e summed over tokens 4i + tau; and the
// matrix-core one (MF true), already combined by the caller: lanes 0-15 hold
// acc[g][j] for d = 8 (lane & 15) + j, the other lanes are ignored.
template <int G, int NT, bool MF>
__device__ void finish_block(const DecodeArgs& a, float (&m_run)[G], float (&l_run)[G], float (&acc)[G][8],
                             unsigned char* wbase, int* s_last, int bh, int b, int h, int split) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int L = tid & 63;
    const int oct = L & 15;
    // ---- wave partial: reduce acc over the 4 token phases (VALU layout), l
    // over lanes
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if constexpr (!MF) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = xor32_sum(xor16_sum(acc[g][e]));
        }
        l_run[g] = wave_sum_dpp(l_run[g]);
    }
    __syncthreads();   // per-wave regions are free now: reuse them for the block merge
    float* wm = reinterpret_cast<float*>(wbase);               // [NW][G]
    float* wl = wm + NW * G;                                   // [NW][G]
    float* wacc = wl + NW * G;                                 // [NW][G][128]
    if (L < 16) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) wacc[(wave * G + g) * 128 + oct * 8 + e] = acc[g][e];
    }
    if (L == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) { wm[wave * G + g] = m_run[g]; wl[wave * G + g] = l_run[g]; }
    }
    __syncthreads();

    // the block's own partial is kept in LDS past the merge scratch
    float* own_ml = reinterpret_cast<float*>(wbase + finish_own_offset(G, NT, a.nsplit));
    float* own_acc = own_ml + 2 * G;
    constexpr int EPT = (G * 128 + NT - 1) / NT;       // acc elements per thread
    float xs[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = tid + e * NT;
        if (i >= G * 128) break;
        const int g = i >> 7, d = i & 127;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w * G + g]);
        float x = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = (wm[w * G + g] == -INFINITY) ? 0.f : exp2f(wm[w * G + g] - M);
            x += wacc[(w * G + g) * 128 + d] * f;
            l += wl[w * G + g] * f;
        }
        xs[e] = x;
        own_acc[i] = x;
        if (d == 0) { own_ml[g] = M; own_ml[G + g] = l; }
    }

    // ---- split merge: every block publishes its partial (device-scope
    // stores), waits until they have completed, then counts itself in; the
    // block that counts last merges all splits (its own partial from LDS).
    {
        float* pml = a.part_ml + ((size_t)bh * a.nsplit + split) * 2 * G;
        float* pacc = a.part_acc + ((size_t)bh * a.nsplit + split) * G * 128;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int i = tid + e * NT;
            if (i >= G * 128) break;
            store_dev(pacc + i, xs[e]);
            if ((i & 127) == 0) { store_dev(pml + (i >> 7), own_ml[i >> 7]); store_dev(pml + G + (i >> 7), own_ml[G + (i >> 7)]); }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.counters + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = (prev == (uint32_t)(a.nsplit - 1));
    }
    __syncthreads();
    if (!*s_last) return;
    merge_splits<G, NT>(a, bh, b, h, reinterpret_cast<float*>(wbase), split, own_ml, own_acc);
    if (tid == 0) __hip_atomic_store(a.counters + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace spark
