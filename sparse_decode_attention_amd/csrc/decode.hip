// Decode attention over the SparK pruned key cache on gfx950 (walkthrough
// section 3.3 and Fig. 3 decode half): every pruned channel of a cached key
// takes the recovery value r_j, then softmax(q K_hat^T * scale) V runs over the
// dense V.
//
// The score is evaluated in its sparse form
//     q . k_hat_t = q . r + sum over kept j of q^j (k_tj - r_j),
// so each token costs G*T multiply-adds instead of G*D.
//
// Work split (flash-decoding style): grid = (nsplit, B*N_kv). A block of 4
// waves owns `chunk` consecutive tokens of one (b, KV head) and all G query
// heads of its group, so every byte of packed K, mask and V is read once per
// step. Each wave walks 64-token tiles, one lane per token for the scores:
//   1. the tile's packed rows (16-byte loads, issued one tile ahead) are
//      staged in LDS; rows whose dword count would be even are padded by one
//      dword so that lanes reading "slot rho of their own row" hit distinct
//      banks;
//   2. each lane turns its mask into the list of table offsets of its T kept
//      channels (a store-only loop over the set bits);
//   3. a uniform loop over the T slots gathers q'_g and r for the slot's
//      channel from an LDS table and accumulates q'_g (k - r): all lanes run
//      the same trip count, so the loads of several slots are in flight
//      together;
//   4. online softmax (base 2, scale folded into q') with wave-wide max;
//   5. P.V with lane = (token mod 4, 8-channel slice of d), 16-byte V loads
//      issued before step 2 so they arrive during the score phase.
// The 4 waves' (m, l, acc) are merged in LDS; the last block of a (b, KV head)
// to finish (device-scope counter) merges all splits, writes the fp32 output
// and resets its counter to zero. Writers never flush their L2: partials go
// out through device-scope stores, and only the merging block invalidates.
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

int tab_stride_for(int G) {
    switch (G) {
        case 1: return (int)sizeof(TabEntry<1>);
        case 2: return (int)sizeof(TabEntry<2>);
        case 4: return (int)sizeof(TabEntry<4>);
        default: return (int)sizeof(TabEntry<8>);
    }
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

DecodeLayout decode_layout(int G, int T, int nsplit, bool sampled, int Tv, bool ragged) {
    DecodeLayout L{};
    L.tab_stride = (uint32_t)tab_stride_for(G);
    // 129 entries (the last one zero: the ragged score loop's filler), then,
    // for the sampled F, the q'_g ns_j table [128][G]
    L.tab_bytes = ((129u * L.tab_stride + 15u) & ~15u) + (sampled ? 128u * (uint32_t)G * 4u : 0u);
    if (ragged) T = 128;      // sized for the longest row
    L.padded = (!ragged && T > 0 && T % 2 == 0 && (T / 2) % 2 == 0) ? 1u : 0u;
    L.half_T = (uint32_t)(T / 2);
    L.magic = L.padded ? (uint32_t)((0x100000000ull + L.half_T - 1) / L.half_T) : 0u;
    if (L.padded) {
        L.row_bytes = (uint32_t)(2 * T + 4);
        L.stage_bytes = (uint32_t)DECODE_TILE * L.row_bytes;
    } else {
        L.row_bytes = (uint32_t)(2 * T);
        // 64 rows plus up to 7 elements of 16-byte misalignment, in whole 16-byte chunks;
        // ragged rows: plus 256 bytes, as a short row's lane reads up to the longest row's length
        L.stage_bytes = (((((uint32_t)DECODE_TILE * (uint32_t)T + 8u) * 2u) + 15u) & ~15u) + (ragged ? 256u : 0u);
    }
    L.list_bytes = (uint32_t)T * DECODE_TILE * 2u;
    L.list_bytes = (L.list_bytes + 15u) & ~15u;
    L.ptab_bytes = (uint32_t)DECODE_TILE * G * 4u;
    // packed V (Tv >= 0): the tile's rows unpadded (up to 7 elements of 16-byte
    // misalignment) plus 256 bytes of slack for the expansion's reads, then
    // the 64 token masks. They are staged after the scores, over the key
    // list and staged keys, so the wave's region is the larger of the two.
    L.vstage_bytes = Tv >= 0 ? ((((uint32_t)DECODE_TILE * (uint32_t)Tv + 8u) * 2u + 15u) & ~15u) + 256u : 0u;
    L.vmask_bytes = Tv >= 0 ? (uint32_t)DECODE_TILE * 16u : 0u;
    L.kv_bytes = L.list_bytes + L.stage_bytes;
    if (L.vstage_bytes + L.vmask_bytes > L.kv_bytes) L.kv_bytes = L.vstage_bytes + L.vmask_bytes;
    L.wave_bytes = L.kv_bytes + L.ptab_bytes;
    const uint32_t waves = DECODE_THREADS / 64;
    uint32_t dyn = waves * L.wave_bytes;
    const uint32_t fin = finish_scratch_bytes(G, DECODE_THREADS, nsplit);
    if (fin > dyn) dyn = fin;
    L.lds_bytes = L.tab_bytes + dyn;
    return L;
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

// Packed rows and mask of one tile, loaded one tile ahead into registers.
struct TileMeta {
    uint4 pk[8];     // up to 8 16-byte chunks per lane (512 per tile)
    uint4 mw;        // this lane's token mask
    size_t ea;       // first loaded element (multiple of 8)
    int shift;       // elements between ea and the tile's first element
    int nchunks;     // 16-byte chunks covering the tile
    int loff;        // ragged rows: the lane's row start within the tile's elements
};

// One packed store: the K cache (packed keys and their masks) or, with V
// channels pruned, the V cache.
struct PackedSrc {
    const uint16_t* packed;   // [B*N_kv][S][T]
    const uint32_t* mask;     // [B*N_kv][S][4]
    size_t elems;             // B*N_kv*S*T
    int T;
};
__device__ __forceinline__ PackedSrc k_src(const DecodeArgs& a) { return {a.packed, a.mask, a.packed_elems, a.T}; }
__device__ __forceinline__ PackedSrc v_src(const DecodeArgs& a) { return {a.v_packed, a.v_mask, a.v_packed_elems, a.Tv}; }

__device__ __forceinline__ uint4 load_chunk(const PackedSrc& p, size_t ce) {
    if (ce + 8 <= p.elems) return *reinterpret_cast<const uint4*>(p.packed + ce);
    uint16_t t[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) t[x] = (ce + x < p.elems) ? p.packed[ce + x] : 0;
    return make_uint4(t[0] | ((uint32_t)t[1] << 16), t[2] | ((uint32_t)t[3] << 16),
                      t[4] | ((uint32_t)t[5] << 16), t[6] | ((uint32_t)t[7] << 16));
}

// S: the head stride in tokens (the cache capacity)
__device__ __forceinline__ void issue_meta(const PackedSrc& p, int S, int bh, int t0, int nt, int L, TileMeta& m) {
    const int T = p.T;
    const size_t e0 = ((size_t)bh * S + t0) * (size_t)T;
    m.ea = e0 & ~(size_t)7;
    m.shift = (int)(e0 - m.ea);
    m.nchunks = T > 0 ? (int)((e0 + (size_t)nt * T - m.ea + 7) >> 3) : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int c = L + 64 * u;
        m.pk[u] = make_uint4(0, 0, 0, 0);
        if (c < m.nchunks) m.pk[u] = load_chunk(p, m.ea + (size_t)c * 8);
    }
    m.mw = make_uint4(0, 0, 0, 0);
    if (L < nt) m.mw = *reinterpret_cast<const uint4*>(p.mask + ((size_t)bh * S + t0 + L) * 4);
}

// Ragged rows (SparK-p): token t of head bh holds its kept values at
// [row_off[t], row_off[t + 1]) of the head's region of S * 128 elements. The
// tile's rows are contiguous; the chunk count is capped at the staging area.
__device__ __forceinline__ void issue_meta_ragged(const DecodeArgs& a, int bh, int t0, int nt, int L, TileMeta& m) {
    const int32_t* ro = a.row_off + (size_t)bh * (a.S + 1);
    const int o0 = ro[t0], o1 = ro[t0 + nt];
    const size_t e0 = (size_t)bh * a.S * 128 + (size_t)o0;
    m.ea = e0 & ~(size_t)7;
    m.shift = (int)(e0 - m.ea);
    const long long n = o1 > o0 ? ((long long)(e0 - m.ea) + (o1 - o0) + 7) >> 3 : 0;
    m.nchunks = (int)min(n, (long long)DECODE_RAGGED_CHUNKS);
    m.loff = L < nt ? ro[t0 + L] - o0 : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int c = L + 64 * u;
        m.pk[u] = make_uint4(0, 0, 0, 0);
        if (c < m.nchunks) m.pk[u] = load_chunk(k_src(a), m.ea + (size_t)c * 8);
    }
    m.mw = make_uint4(0, 0, 0, 0);
    if (L < nt) m.mw = *reinterpret_cast<const uint4*>(a.mask + ((size_t)bh * a.S + t0 + L) * 4);
}

// Write one 16-byte chunk c of the tile into the staged rows.
__device__ __forceinline__ void stage_chunk(const DecodeLayout& lay, const TileMeta& m, int c, uint4 x,
                                            unsigned char* stage, int tile_dwords) {
    if (!lay.padded) {
        reinterpret_cast<uint4*>(stage)[c] = x;
        return;
    }
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int u = 4 * c + i - (m.shift >> 1);          // dword index within the tile (T even)
        if (u >= 0 && u < tile_dwords) {
            const uint32_t row = __umulhi((uint32_t)u, lay.magic);
            reinterpret_cast<uint32_t*>(stage)[u + row] = w4[i];
        }
    }
}

// Online softmax over one 64-token tile (base 2): lane L holds the scores of
// token L for the G heads; p goes to ptab[L][g] and the running (m, l) and
// the P.V accumulators are rescaled.
template <int G>
__device__ __forceinline__ void softmax_tile(const float (&s)[G], float (&m_run)[G], float (&l_run)[G],
                                             float (&acc)[G][8], float* ptab, int L) {
    float alpha[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mt = wave_max_dpp(s[g]);
        const float mn = fmaxf(m_run[g], mt);
        // hardware exp2 (v_exp_f32, about 1 ulp, no denormal rescaling):
        // both arguments are <= 0, so every value is at most 1
        alpha[g] = __builtin_amdgcn_exp2f(m_run[g] - mn);
        const float p = __builtin_amdgcn_exp2f(s[g] - mn);
        l_run[g] = l_run[g] * alpha[g] + p;
        m_run[g] = mn;
        ptab[L * G + g] = p;
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] *= alpha[g];
}

// P.V of one tile: lane (tau, oct) holds V rows 4i+tau, d in [8 oct, 8 oct + 8).
template <int G>
__device__ __forceinline__ void pv_tile(const uint4 (&vr)[16], const float* ptab, float (&acc)[G][8], int tau) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        // p rows are read four at a time: reading all 16 ahead would hold
        // 16 * G registers on top of the V tile
        if ((i & 3) == 0) __builtin_amdgcn_sched_barrier(0);
        const int tok = 4 * i + tau;
        const QRow<G> p = *reinterpret_cast<const QRow<G>*>(ptab + tok * G);
        const uint32_t w4[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
        float vf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vf[2 * e] = bf16_lo(w4[e]);
            vf[2 * e + 1] = bf16_hi(w4[e]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p.v[g], vf[e], acc[g][e]);
    }
}

// P.V of one tile over a packed V cache (V channels pruned): lane (tau, oct)
// expands, for each of its rows 4i + tau, the 8 channels d in [8 oct, 8 oct + 8)
// from the staged packed row. Those channels' retained values are contiguous
// in the row (ascending channel order), starting at the number of kept
// channels below 8 oct; a pruned channel takes its recovery value rv (fp32).
// Every read stays inside the staged tile plus its slack: the rank is below
// the number of set mask bits, at most 128.
template <int G>
__device__ __forceinline__ void pv_tile_vpacked(const uint16_t* vst, const uint4* vmask, int Tv, const float* ptab,
                                                const float (&rvl)[8], float (&acc)[G][8], int tau, int oct) {
    const int wsel = oct >> 2;
    const uint32_t sh = 8u * (uint32_t)(oct & 3);
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
        const int tok = 4 * i + tau;
        const uint4 mw = vmask[tok];
        const uint32_t word = wsel == 0 ? mw.x : wsel == 1 ? mw.y : wsel == 2 ? mw.z : mw.w;
        uint32_t idx = (wsel > 0 ? __popc(mw.x) : 0u) + (wsel > 1 ? __popc(mw.y) : 0u) +
                       (wsel > 2 ? __popc(mw.z) : 0u) + __popc(word & ((1u << sh) - 1u));
        const uint32_t bits = (word >> sh) & 0xFFu;
        const uint16_t* row = vst + tok * Tv;
        const QRow<G> p = *reinterpret_cast<const QRow<G>*>(ptab + tok * G);
        float vf[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool kept = (bits >> e) & 1u;
            const float x = bf16_to_f32(row[idx]);
            vf[e] = kept ? x : rvl[e];
            idx += kept ? 1u : 0u;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(p.v[g], vf[e], acc[g][e]);
    }
}

// V rows of one tile for the P.V layout: lane (tau, oct) takes rows 4i + tau,
// d in [8 oct, 8 oct + 8). Rows past the end of a partial tile re-read the
// last valid row; their p is 0.
__device__ __forceinline__ void load_v_tile(const uint16_t* vbh, int t0, int nt, int tau, int oct, uint4 (&vr)[16]) {
    // 32-bit byte offsets from the head's V slab (at most 64K rows of 256 B),
    // so each request is a scalar base plus one vector offset
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(vbh);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t row = (uint32_t)(t0 + min(4 * i + tau, nt - 1));
        vr[i] = *reinterpret_cast<const uint4*>(vb + (row * 256u + (uint32_t)oct * 16u));
    }
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
// matrix-core one (MF true), where acc[g][j] is row g (lanes 0-15: hi part of
// p) or row 4 + g (lanes 16-31: lo part) of the 16x16 tile j, column
// d = 8 (lane & 15) + j; lanes 32-63 hold zero rows.
template <int G, int NT, bool MF>
__device__ void finish_block(const DecodeArgs& a, float (&m_run)[G], float (&l_run)[G], float (&acc)[G][8],
                             unsigned char* wbase, int* s_last, int bh, int b, int h, int split) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int L = tid & 63;
    const int oct = L & 15;
    // ---- wave partial: reduce acc over the 4 token phases (or add the hi
    // and lo rows), l over lanes
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = MF ? xor16_sum(acc[g][e]) : xor32_sum(xor16_sum(acc[g][e]));
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

// SMODE: 0 for the recovery vector r, else the sampled F (4 Gaussian,
// 5 Exponential). Sampled F, G <= 4: two waves per SIMD (it fits without
// spills), so the Philox and sample arithmetic of one wave covers the
// latency of the other.
//
// VP: the V cache is packed too (V channels pruned): its rows and masks are
// loaded one tile ahead like the keys', staged in LDS, and expanded in P.V.
//
// RG: ragged packed rows (SparK-p): per-lane row starts and counts; the score
// loop runs to the wave's longest row, shorter rows pointing their surplus
// slots at a zero table entry and reading 0 for their values.
template <int G, int SMODE, bool VP, bool RG>
__global__ void __launch_bounds__(DECODE_THREADS) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 2 : 1)))
decode_kernel(const DecodeArgs a) {
    constexpr bool SAMPLED = SMODE != 0;
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = DECODE_THREADS / 64;
    const DecodeLayout& lay = a.lay;
    unsigned char* tab = smem;                                 // [128] x tab_stride: q'_0..q'_{G-1}, r
    unsigned char* wbase = smem + lay.tab_bytes;

    const int bh = blockIdx.y;
    const int split = blockIdx.x;
    const int N_kv = a.N_kv;
    const int b = bh / N_kv, h = bh % N_kv;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int L = tid & 63;
    const int S = a.S, T = RG ? 128 : a.T;
    constexpr uint32_t TAB = (uint32_t)sizeof(TabEntry<G>);
    const bool even_T = !RG && (T % 2) == 0;

    // ---- table of q' (q * scale * log2 e) and r per channel. Sampled F: r
    // holds (mu, sigma); a pruned key is w / a_j, a_j = sqrt(A_j), with the
    // sample w = mu + ns n: the table takes r_j = mu / a_j and, in a second
    // table, q'_g ns / a_j (ns = sigma for the Gaussian, mu for the Exponential)
    float* qn = reinterpret_cast<float*>(tab + ((129 * TAB + 15) & ~15u));   // [128][G], sampled F only
    for (int i = tid; i < 128 * G; i += DECODE_THREADS) {
        const int g = i >> 7, j = i & 127;
        const uint16_t qb = a.q[((size_t)b * a.N_q + (size_t)h * G + g) * 128 + j];
        const float qv = bf16_to_f32(qb) * a.qscale;
        reinterpret_cast<TabEntry<G>*>(tab)[j].q[g] = qv;
        if (SAMPLED) {
            const float Aj = a.A[(size_t)bh * 128 + j];
            const float inv_a = Aj > 0.0f ? 1.0f / sqrtf(Aj) : 0.0f;
            const float ns = a.r[(size_t)bh * 128 + (SMODE == 4 ? 1 : 0)];
            qn[j * G + g] = qv * (ns * inv_a);
            if (g == 0) reinterpret_cast<TabEntry<G>*>(tab)[j].r = a.r[(size_t)bh * 128] * inv_a;
        }
    }
    if (!SAMPLED && tid < 128) reinterpret_cast<TabEntry<G>*>(tab)[tid].r = a.r[(size_t)bh * 128 + tid];
    if (tid < (int)(TAB / 4)) reinterpret_cast<float*>(tab + 128 * TAB)[tid] = 0.0f;     // the zero entry

    uint16_t* lst = reinterpret_cast<uint16_t*>(wbase + (size_t)wave * lay.wave_bytes);     // [T][64]
    unsigned char* stage = wbase + (size_t)wave * lay.wave_bytes + lay.list_bytes;
    float* ptab = reinterpret_cast<float*>(wbase + (size_t)wave * lay.wave_bytes + lay.kv_bytes);   // [64][G]
    // VP: packed V rows and masks, over the list and staged keys (dead after the scores)
    unsigned char* vstage = wbase + (size_t)wave * lay.wave_bytes;
    uint4* vmask = reinterpret_cast<uint4*>(vstage + lay.vstage_bytes);                  // [64] V masks
    // every list entry holds a valid table offset from the start
    for (int rho = 0; rho < T; ++rho) lst[rho * 64 + L] = 0;
    __syncthreads();

    // c_g = q'_g . r: the score of a key whose channels are all pruned
    float cq[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const TabEntry<G>* te = reinterpret_cast<const TabEntry<G>*>(tab);
        cq[g] = wave_sum(te[L].q[g] * te[L].r + te[L + 64].q[g] * te[L + 64].r);
    }

    const int blk_begin = split * a.chunk;
    const int blk_end = min(S, blk_begin + a.chunk);
    const int ntiles = (blk_end - blk_begin + DECODE_TILE - 1) / DECODE_TILE;

    const int tau = L >> 4;        // token phase in the P.V layout
    const int oct = L & 15;        // 8-channel slice of d

    float m_run[G], l_run[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m_run[g] = -INFINITY;
        l_run[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    }

    const uint16_t* vbh = VP ? nullptr : a.v + (size_t)bh * a.S_cap * 128;
    float rvl[8];          // VP: recovery values of this lane's 8 V channels
    if (VP) {
#pragma unroll
        for (int e = 0; e < 8; ++e) rvl[e] = a.rv[(size_t)bh * 128 + oct * 8 + e];
    }

    TileMeta meta, vmeta;
    if (wave < ntiles) {
        const int t0 = blk_begin + wave * DECODE_TILE;
        if (RG) issue_meta_ragged(a, bh, t0, min(DECODE_TILE, blk_end - t0), L, meta);
        else issue_meta(k_src(a), a.S_cap, bh, t0, min(DECODE_TILE, blk_end - t0), L, meta);
        if (VP) issue_meta(v_src(a), a.S_cap, bh, t0, min(DECODE_TILE, blk_end - t0), L, vmeta);
    }

    for (int tile = wave; tile < ntiles; tile += NW) {
        const int t0 = blk_begin + tile * DECODE_TILE;
        const int nt = min(DECODE_TILE, blk_end - t0);

        // -- 1. stage this tile's packed rows (loaded one tile ahead)
        if (RG || T > 0) {
            const int tile_dwords = (nt * T) >> 1;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int c = L + 64 * u;
                if (c < meta.nchunks) stage_chunk(lay, meta, c, meta.pk[u], stage, tile_dwords);
            }
            for (int c = L + 512; c < meta.nchunks; c += 64)      // rows longer than 64 elements
                stage_chunk(lay, meta, c, load_chunk(k_src(a), meta.ea + (size_t)c * 8), stage, tile_dwords);
        }
        const uint4 mw = meta.mw;
        const int row_base = RG ? 2 * (meta.shift + meta.loff)
                                : (lay.padded ? 0 : 2 * meta.shift) + L * (int)lay.row_bytes;

        // -- V of this tile (dense V), then the next tile's packed keys and mask
        uint4 vr[16];
        if (!VP) load_v_tile(vbh, t0, nt, tau, oct, vr);
        if (tile + NW < ntiles) {
            const int t1 = t0 + NW * DECODE_TILE;
            if (RG) issue_meta_ragged(a, bh, t1, min(DECODE_TILE, blk_end - t1), L, meta);
            else issue_meta(k_src(a), a.S_cap, bh, t1, min(DECODE_TILE, blk_end - t1), L, meta);
        }

        // -- 2. list of kept channels (table byte offsets), slot-major [rho][lane]
        int nslots = T;     // ragged rows: the wave's longest row
        int cnt = 0;        // this lane's kept channels
        {
            const uint32_t words[4] = {mw.x, mw.y, mw.z, mw.w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t m = words[w];
                while (m) {
                    const uint32_t j = 32u * w + (uint32_t)__builtin_ctz(m);
                    m &= m - 1;
                    lst[cnt * 64 + L] = (uint16_t)(j * TAB);
                    ++cnt;
                }
            }
            if (RG) {
                nslots = (int)__builtin_amdgcn_readfirstlane((uint32_t)wave_max_dpp((float)cnt));
                for (int rho = cnt; rho < nslots; ++rho) lst[rho * 64 + L] = (uint16_t)(128u * TAB);
            }
        }
        wave_lds_sync();

        // -- 3. scores, one lane per token, 8 slots per batch: the 8 list
        //       entries, then the 8 table rows and packed values, are each
        //       requested together before any of them is used
        float s[G];
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = 0.f;
        {
            const uint16_t* lrow = lst + L;
            const unsigned char* krow = stage + row_base;
            const int T8 = nslots & ~7;
            for (int rho = 0; rho < T8; rho += 8) {
                uint32_t off[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) off[k] = lrow[(rho + k) * 64];
                float kv[8];
                if (RG) {
                    // slots past this lane's row read other rows or unwritten
                    // memory: their values are replaced by 0 (q' is 0 there too)
                    const uint16_t* k16 = reinterpret_cast<const uint16_t*>(krow + 2 * rho);
#pragma unroll
                    for (int k = 0; k < 8; ++k) kv[k] = rho + k < cnt ? bf16_to_f32(k16[k]) : 0.0f;
                } else if (even_T) {
                    // rows start 4-byte aligned when T is even: two bf16 per dword read
                    const uint32_t* k32 = reinterpret_cast<const uint32_t*>(krow + 2 * rho);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t two = k32[k];
                        kv[2 * k] = bf16_lo(two);
                        kv[2 * k + 1] = bf16_hi(two);
                    }
                } else {
                    const uint16_t* k16 = reinterpret_cast<const uint16_t*>(krow + 2 * rho);
#pragma unroll
                    for (int k = 0; k < 8; ++k) kv[k] = bf16_to_f32(k16[k]);
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const TabEntry<G>& te = *reinterpret_cast<const TabEntry<G>*>(
                        __builtin_assume_aligned(tab + off[k], 16));
                    const float e = kv[k] - te.r;
#pragma unroll
                    for (int g = 0; g < G; ++g) s[g] = fmaf(te.q[g], e, s[g]);
                }
            }
            for (int rho = T8; rho < nslots; ++rho) {
                const TabEntry<G>& te = *reinterpret_cast<const TabEntry<G>*>(
                    __builtin_assume_aligned(tab + lrow[rho * 64], 16));
                const float kx = bf16_to_f32(*reinterpret_cast<const uint16_t*>(krow + 2 * rho));
                const float e = (RG && rho >= cnt ? 0.0f : kx) - te.r;
#pragma unroll
                for (int g = 0; g < G; ++g) s[g] = fmaf(te.q[g], e, s[g]);
            }
        }
        if (SAMPLED) sampled_scores<G, SMODE == 4>(a, qn, mw, bh, t0, nt, L, s);
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = (L < nt) ? s[g] + cq[g] : -INFINITY;

        // -- 4. online softmax (base 2)
        softmax_tile<G>(s, m_run, l_run, acc, ptab, L);
        wave_lds_sync();

        int vshift = 0;
        if (VP) {
            // packed V rows (16-byte chunks as loaded) and the tile's V masks,
            // over the list and staged keys; then the next tile's V rows
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int c = L + 64 * u;
                if (c < vmeta.nchunks) reinterpret_cast<uint4*>(vstage)[c] = vmeta.pk[u];
            }
            for (int c = L + 512; c < vmeta.nchunks; c += 64)
                reinterpret_cast<uint4*>(vstage)[c] = load_chunk(v_src(a), vmeta.ea + (size_t)c * 8);
            vmask[L] = vmeta.mw;
            vshift = vmeta.shift;
            if (tile + NW < ntiles) {
                const int t1 = t0 + NW * DECODE_TILE;
                issue_meta(v_src(a), a.S_cap, bh, t1, min(DECODE_TILE, blk_end - t1), L, vmeta);
            }
            wave_lds_sync();
        }

        // -- 5. P.V
        if (VP)
            pv_tile_vpacked<G>(reinterpret_cast<const uint16_t*>(vstage) + vshift, vmask, a.Tv, ptab, rvl, acc, tau,
                               oct);
        else
            pv_tile<G>(vr, ptab, acc, tau);
        wave_lds_sync();
    }

    __shared__ int s_last;
    finish_block<G, DECODE_THREADS, false>(a, m_run, l_run, acc, wbase, &s_last, bh, b, h, split);
}

// Mask and packed row of token t0 + min(L, nt - 1): lanes past the end of a
// partial tile re-read the last valid row (their scores are discarded).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Slot of token t (0..63) in a ptab row: within each 16-token group the
// token 16 grp + 4 e + tau sits at 16 grp + 4 tau + e, so the four tokens
// that one lane of the matrix-core P.V needs are adjacent.
__device__ __forceinline__ uint32_t ptab_slot(uint32_t t) { return (t & 48u) | ((t & 3u) << 2) | ((t >> 2) & 3u); }

// Online softmax of one tile for the matrix-core P.V: p goes to ptab as
// [g][64 token slots] fp32; accm[j][g] (the rows of head g) are rescaled.
template <int G>
__device__ __forceinline__ void softmax_tile_mf(const float (&s)[G], float (&m_run)[G], float (&l_run)[G],
                                                f32x4 (&accm)[8], float* ptab, int L) {
    static_assert(G == 4, "one accumulator row per head");
    f32x4 alpha;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mt = wave_max_dpp(s[g]);
        const float mn = fmaxf(m_run[g], mt);
        // hardware exp2 (v_exp_f32, about 1 ulp, no denormal rescaling):
        // both arguments are <= 0, so every value is at most 1
        alpha[g] = __builtin_amdgcn_exp2f(m_run[g] - mn);
        const float p = __builtin_amdgcn_exp2f(s[g] - mn);
        l_run[g] = l_run[g] * alpha[g] + p;
        m_run[g] = mn;
        ptab[g * 64 + ptab_slot((uint32_t)L)] = p;
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) accm[nb] *= alpha;
}

// P.V of one 64-token tile on the matrix cores (v_mfma_f32_16x16x16_bf16,
// four heads), with V taken from the registers it was loaded into: lane
// (tau, oct) holds vr[i] = V row 4i + tau, d in [8 oct, 8 oct + 8). Per
// 16-token group grp and column offset j (0..7), with K index k = 4 tau + e
// standing for token 16 grp + 4 e + tau:
//   A (16 x 16): row g < 4 is bf16(p_g), row 4 + g is bf16(p_g - bf16(p_g)),
//                rows 8-15 are zero, so the hi and lo rows carry p to ~2^-16;
//   B (16 x 16): B[k][n] = V[token(k)][8 n + j], element j of
//                vr[4 grp + e] in lane (tau, n), two byte permutes per MFMA;
//   D (16 x 16): accm[j]; lane l holds rows 4 (l >> 4) + e (hi rows in lanes
//                0-15, lo rows in lanes 16-31), column n = l & 15, i.e.
//                d = 8 (l & 15) + j.
// No V bytes go through LDS.
__device__ __forceinline__ uint32_t dword_of(const uint4& x, int j) {
    return j == 0 ? x.x : j == 1 ? x.y : j == 2 ? x.z : x.w;
}
__device__ __forceinline__ void pv_tile_mf(const uint4 (&vr)[16], const float* ptab, f32x4 (&accm)[8], int L) {
    const uint32_t m = (uint32_t)L & 15u, q = (uint32_t)L >> 4;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
        const float4 pv = *reinterpret_cast<const float4*>(ptab + (m & 3u) * 64u + 16u * grp + 4u * q);
        const uint32_t hi0 = pack_bf16(pv.x, pv.y), hi1 = pack_bf16(pv.z, pv.w);
        const uint32_t lo0 = pack_bf16(pv.x - bf16_lo(hi0), pv.y - bf16_hi(hi0));
        const uint32_t lo1 = pack_bf16(pv.z - bf16_lo(hi1), pv.w - bf16_hi(hi1));
        const u32x2 aw = {m < 4u ? hi0 : (m < 8u ? lo0 : 0u), m < 4u ? hi1 : (m < 8u ? lo1 : 0u)};
        const i16x4 av = __builtin_bit_cast(i16x4, aw);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // bf16 element j of four V rows: low halves for even j, high for odd
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            const u32x2 bw = {__builtin_amdgcn_perm(dword_of(vr[4 * grp + 1], j >> 1), dword_of(vr[4 * grp], j >> 1), sel),
                              __builtin_amdgcn_perm(dword_of(vr[4 * grp + 3], j >> 1), dword_of(vr[4 * grp + 2], j >> 1), sel)};
            accm[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(i16x4, bw), accm[j], 0, 0, 0);
        }
    }
}

template <int T>
__device__ __forceinline__ void load_row(const DecodeArgs& a, int bh, int t0, int nt, int L,
                                         uint4& mw, uint32_t (&kr)[(T + 1) / 2]) {
    constexpr int NDW = (T + 1) / 2;
    const size_t row = (size_t)bh * a.S_cap + t0 + min(L, nt - 1);
    mw = *reinterpret_cast<const uint4*>(a.mask + row * 4);
    if constexpr (T % 8 == 0) {
        const uint4* src = reinterpret_cast<const uint4*>(a.packed + row * T);   // 16-byte aligned rows
#pragma unroll
        for (int i = 0; i < NDW / 4; ++i) {
            const uint4 x = src[i];
            kr[4 * i] = x.x; kr[4 * i + 1] = x.y; kr[4 * i + 2] = x.z; kr[4 * i + 3] = x.w;
        }
    } else {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.packed + row * T);  // 4-byte aligned rows
#pragma unroll
        for (int i = 0; i < NDW; ++i) kr[i] = src[i];
    }
}

// Ragged rows (SparK-p): the row of lane L's token starts at element o of the
// head's packed region (S * 128 elements) and holds c = oe - o values. The
// lane requests the 65 dwords from the one holding element o on (sixteen
// 16-byte requests and one dword, no branches), so kr[i] holds slots 2 i - sh
// and 2 i - sh + 1 (sh = o & 1); what lies past the row is never used. A lane
// whose 65 dwords would leave the region (a row near the end of a nearly full
// region, which may end the allocation) requests the region's first 65
// instead and then, in a branch taken only when the wave has such a lane,
// exactly its row's dwords, one by one.
constexpr int RAGGED_KR = 65;
struct RaggedRows {
    int sh, c;        // this tile's row: element shift and count
    int o_nx, oe_nx;  // offsets of the next tile's row (requested a tile ahead)
};
__device__ __forceinline__ void ragged_offsets(const DecodeArgs& a, int bh, int t, int& o, int& oe) {
    const int32_t* ro = a.row_off + (size_t)bh * (a.S + 1);
    o = ro[t];
    oe = ro[t + 1];
}
__device__ __forceinline__ void load_row_ragged(const DecodeArgs& a, int bh, int t, int o, int oe, uint4& mw,
                                                uint32_t (&kr)[RAGGED_KR], RaggedRows& rr) {
    typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
    mw = *reinterpret_cast<const uint4*>(a.mask + ((size_t)bh * a.S + t) * 4);
    const int c = min(max(oe - o, 0), 128);
    rr.sh = o & 1;
    rr.c = c;
    const int ndw = (rr.sh + c + 1) >> 1;
    const int o_dw = o >> 1;
    const bool near_end = o_dw + RAGGED_KR > a.S * 64;
    const uint32_t* head = reinterpret_cast<const uint32_t*>(a.packed + (size_t)bh * a.S * 128);
    const uint32_t* src = head + (near_end ? 0 : o_dw);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const u32x4_a4 x = *reinterpret_cast<const u32x4_a4*>(src + 4 * i);
        kr[4 * i] = x.x; kr[4 * i + 1] = x.y; kr[4 * i + 2] = x.z; kr[4 * i + 3] = x.w;
    }
    kr[64] = src[64];
    if (ballot(near_end) != 0) {
        if (near_end) {
            const uint32_t* row = head + o_dw;
#pragma unroll
            for (int i = 0; i < RAGGED_KR; ++i)
                if (i < ndw) kr[i] = row[i];
        }
    }
}

// Row stride (u16 elements) of the lane-major slot list: room for T slots and
// a spare one, rounded so that the stride in dwords is odd, which puts the 64
// lanes of a dword read on distinct bank pairs.
__host__ __device__ constexpr uint32_t list_stride_of(int T) {
    return ((T / 2) % 2 == 1) ? (uint32_t)T + 2u : (uint32_t)T + 4u;
}
template <int T>
constexpr uint32_t list_stride() { return list_stride_of(T); }
// LDS bytes of one wave's slot list, in whole 16-byte units
__host__ __device__ constexpr uint32_t list_bytes_of(int T) { return (64u * list_stride_of(T) * 2u + 15u) & ~15u; }

// Slot list of one tile, lane-major: lst[lane * stride + rho] = 4 * c for the
// lane's rho-th kept channel c (ascending), i.e. the byte offset of c's r in
// the fast kernel's r table (a quarter of the offset of its q' row). One
// bit-clearing loop per mask word; lanes leave it as their word empties.
template <int T>
__device__ __forceinline__ void build_list(const uint4& mw, uint8_t* lst, int L) {
    uint16_t* p = reinterpret_cast<uint16_t*>(lst) + (uint32_t)L * list_stride<T>();
    const uint32_t words[4] = {mw.x, mw.y, mw.z, mw.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t m = words[w];
        const int pc = __builtin_popcount(m);
        int i = 0;
        // four bits per trip while at least four remain, then one at a time
        for (; i + 4 <= pc; i += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                p[i + u] = (uint16_t)(((uint32_t)__builtin_ctz(m) << 2) | (128u * w));
                m &= m - 1;
            }
        }
        for (; i < pc; ++i) {
            p[i] = (uint16_t)(((uint32_t)__builtin_ctz(m) << 2) | (128u * w));
            m &= m - 1;
        }
        p += pc;
    }
}

// One 64-token tile of the fast kernel. The slot list is built from the
// tile's mask (before the call when LIST_READY); then the tile's V rows are
// requested (unless LOAD_V is false: then the prologue did), so they arrive
// during the score loop and the softmax; the next tile's mask and packed
// rows are requested once the scores have consumed this tile's; then P.V.
// A request made while the memory queue is full stalls the wave, so none is
// placed ahead of work that needs no memory.
//
// RG (ragged rows, T = 128): the score loop runs to the wave's longest row,
// and a slot past its lane's row adds nothing (its list entry is a stale but
// valid table offset, its value is discarded). The offsets of the tile after
// next are requested once the next tile's rows are (nt_next2 tokens).
template <int G, int T, int SMODE, bool LOAD_V, bool LIST_READY, bool RG = false>
__device__ __forceinline__ void fast_tile(const DecodeArgs& a, int bh, const unsigned char* tab, uint8_t* lst,
                                          float* ptab, const uint16_t* vbh, const float (&cq)[G], int t0, int nt,
                                          int nt_next, int L, uint4& mw,
                                          uint32_t (&kr)[RG ? RAGGED_KR : (T + 1) / 2], uint4 (&vr)[16],
                                          float (&m_run)[G], float (&l_run)[G], f32x4 (&accm)[8], const float* qn,
                                          RaggedRows& rr, int nt_next2) {
    const int tau = L >> 4, oct = L & 15;
    const int t1 = t0 + (DECODE_FAST_THREADS / 64) * DECODE_TILE;
    if constexpr (!LIST_READY) build_list<T>(mw, lst, L);
    if constexpr (LOAD_V) load_v_tile(vbh, t0, nt, tau, oct, vr);
    wave_lds_sync();
    // scores: s_g = q'_g . r + sum over kept c of q'_g(c) (k_c - r_c), with
    // q' = q * scale * log2(e) as fp32 float4 per channel (tab) and r as fp32
    // per channel (rtab, 2 KiB after tab); slots in batches of NB: the
    // batch's q' rows and r values, then its FMAs
    static_assert(G == 4, "table row holds four heads");
    const uint16_t* lrow16 = reinterpret_cast<const uint16_t*>(lst) + (uint32_t)L * list_stride<T>();
    const unsigned char* rtab = tab + 128 * 16;
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = cq[g];
    // ragged rows: slots up to the wave's longest row (a wave-uniform bound)
    const int nmax = RG ? (int)wave_max_dpp((float)rr.c) : T;
    const uint32_t sh16 = RG ? 16u * (uint32_t)rr.sh : 0u;
    // (batches of 4 for ragged rows: that variant holds 65 row registers and
    // otherwise spills)
    constexpr int NB = RG ? 4 : 8;
    // the list entries of each batch are requested one batch ahead, so their
    // LDS round trip overlaps the previous batch's gathers
    uint32_t off_next[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k)
        if (k < T) off_next[k] = lrow16[k];
#pragma unroll
    for (int r0 = 0; r0 < T; r0 += NB) {
        // (ragged rows: batches past the longest row are skipped, uniformly)
        if (RG && r0 >= nmax) continue;
        // keep each batch's loads inside the batch: unbounded hoisting across
        // the fully unrolled slot loop would need registers for every slot
        __builtin_amdgcn_sched_barrier(0);
        uint32_t off[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) off[k] = off_next[k];
#pragma unroll
        for (int k = 0; k < NB; ++k)
            if (r0 + NB + k < T) off_next[k] = lrow16[r0 + NB + k];
        float4 qv[NB];
        float rv[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (r0 + k < T) {
                qv[k] = *reinterpret_cast<const float4*>(__builtin_assume_aligned(tab + 4u * off[k], 16));
                rv[k] = *reinterpret_cast<const float*>(rtab + off[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (r0 + k < T) {
                const int rho = r0 + k;
                float kv;
                if constexpr (RG) {
                    // slots rho & ~1 and rho | 1 of the row, whatever its shift
                    const uint32_t w = __builtin_amdgcn_alignbit(kr[(rho >> 1) + 1], kr[rho >> 1], sh16);
                    kv = (rho & 1) ? bf16_hi(w) : bf16_lo(w);
                } else {
                    kv = (rho & 1) ? bf16_hi(kr[rho >> 1]) : bf16_lo(kr[rho >> 1]);
                }
                float e = kv - rv[k];
                if (RG) e = rho < rr.c ? e : 0.0f;
                s[0] = fmaf(qv[k].x, e, s[0]);
                s[1] = fmaf(qv[k].y, e, s[1]);
                s[2] = fmaf(qv[k].z, e, s[2]);
                s[3] = fmaf(qv[k].w, e, s[3]);
            }
        }
        // consume the partial sums here: otherwise the compiler sinks the
        // FMAs of every batch to the end and keeps all gathered rows live
#pragma unroll
        for (int g = 0; g < G; ++g) asm volatile("" : "+v"(s[g]));
    }
    // sampled F: the sample term needs this tile's mask, so it runs before
    // the next tile's masks are requested into mw
    if (SMODE) sampled_scores<G, SMODE == 4>(a, qn, mw, bh, t0, nt, L, s);
    if (L >= nt) {
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = -INFINITY;
    }
    // the packed rows are consumed: request the next tile's into them
    if constexpr (RG) {
        if (nt_next > 0) {
            load_row_ragged(a, bh, t1 + min(L, nt_next - 1), rr.o_nx, rr.oe_nx, mw, kr, rr);
            if (nt_next2 > 0)
                ragged_offsets(a, bh, t1 + (DECODE_FAST_THREADS / 64) * DECODE_TILE + min(L, nt_next2 - 1), rr.o_nx,
                               rr.oe_nx);
        }
    } else {
        if (nt_next > 0) load_row<T>(a, bh, t1, nt_next, L, mw, kr);
    }
    softmax_tile_mf<G>(s, m_run, l_run, accm, ptab, L);
    wave_lds_sync();
    pv_tile_mf(vr, ptab, accm, L);
    wave_lds_sync();
}

// Decode block specialised for a compile-time T (the pruning ratios in use):
// DECODE_FAST_THREADS threads (8 waves) per block, one block per CU. Each
// lane loads its token's packed row straight into registers (T/2 dwords, no
// LDS staging) and builds the list of its kept channels in LDS as u16 table
// offsets; the score loop then knows each slot's register at compile time.
//
// SMODE 4 / 5: the sampled F (Gaussian / Exponential); the r table then holds
// mu / a_j, and a q' ns table of 2 KiB follows the other LDS.
//
// RG: ragged rows (SparK-p, T = 128 slots): row offsets are read a tile
// ahead, each lane's row goes into 65 registers (load_row_ragged).
template <int G, int T, int SMODE, bool RG = false>
__global__ void __launch_bounds__(DECODE_FAST_THREADS)
decode_fast_kernel(const DecodeArgs a) {
    // statically sized LDS: its base address is a compile-time constant, so
    // table offsets fold into the LDS instructions' offset fields
    constexpr uint32_t LDS = RG ? DECODE_FAST_RAGGED_LDS_BYTES : DECODE_FAST_LDS_BYTES;
    __shared__ __align__(16) unsigned char smem[LDS + (SMODE ? 128 * G * 4 : 0)];
    float* qn = reinterpret_cast<float*>(smem + LDS);   // [128][G], sampled F only
    // tables: q'_0..q'_3 of the group as a float4 per channel (2 KiB), then
    // r as one float per channel (512 bytes)
    constexpr uint32_t TAB = 16u;
    constexpr uint32_t TABLES = 128u * 16u + 128u * 4u;     // then a 16-byte flag slot
    // per wave: the slot list (u16, lane-major), then p as [G][64] fp32
    constexpr uint32_t LIST = list_bytes_of(T);
    constexpr uint32_t WAVE = LIST + 64u * G * 4u;
    constexpr int NW = DECODE_FAST_THREADS / 64;
    static_assert(RG ? (T == 128 && SMODE == 0) : (T % 2 == 0 && T > 0 && T < 128),
                  "fast path needs an even 0 < T < 128, or 128 slots for ragged rows");
    constexpr int KR = RG ? RAGGED_KR : (T + 1) / 2;
    unsigned char* tab = smem;
    unsigned char* wbase = smem + TABLES + 16;

    const int bh = blockIdx.y;
    const int split = blockIdx.x;
    const int b = bh / a.N_kv, h = bh % a.N_kv;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int L = tid & 63;
    const int S = a.S;
    const int blk_begin = split * a.chunk;
    const int blk_end = min(S, blk_begin + a.chunk);
    const int ntiles = (blk_end - blk_begin + DECODE_TILE - 1) / DECODE_TILE;

    // Request order and timing matter. With the whole first tile of every
    // wave requested at once (about 200 KB per CU), any single request takes
    // as long as that flood takes to drain. So: q and r first; then (after a
    // barrier, so that every wave has requested q and r) the packed rows and
    // masks of the first tile; the V rows only once this wave's masks have
    // arrived. The slot list and the table are built while the packed rows
    // and V rows stream in. The loads are unconditional (indices clamped into
    // the head) so that no register copy makes a wave wait early.
    static_assert((128 * G) % DECODE_FAST_THREADS == 0, "q values per thread");
    constexpr int QPT = 128 * G / DECODE_FAST_THREADS;
    uint16_t qb[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int j = tid + i * DECODE_FAST_THREADS;
        qb[i] = a.q[((size_t)b * a.N_q + (size_t)h * G + (j >> 7)) * 128 + (j & 127)];
    }
    float rv = a.r[(size_t)bh * 128 + (tid & 127)];
    float ns = 0.0f;     // sampled F: the noise scale of channel tid & 127 back-solved
    if (SMODE) {
        // r holds (mu, sigma); a pruned key is (mu + ns n) / a_j, a_j = sqrt(A_j)
        const float Aj = a.A[(size_t)bh * 128 + (tid & 127)];
        const float inv_a = Aj > 0.0f ? 1.0f / sqrtf(Aj) : 0.0f;
        const float mu = a.r[(size_t)bh * 128], sigma = a.r[(size_t)bh * 128 + 1];
        rv = mu * inv_a;
        ns = (SMODE == 4 ? sigma : mu) * inv_a;
    }
    // ragged rows: the first tile's row offsets are requested with q and r,
    // the second tile's right after them
    RaggedRows rr{};
    int o0 = 0, oe0 = 0;
    if constexpr (RG) {
        const int tr0 = min(blk_begin + wave * DECODE_TILE, S - 1);
        ragged_offsets(a, bh, tr0 + min(L, max(1, min(DECODE_TILE, blk_end - tr0)) - 1), o0, oe0);
        const int t1 = blk_begin + (wave + NW) * DECODE_TILE;
        if (t1 < blk_end) ragged_offsets(a, bh, t1 + min(L, min(DECODE_TILE, blk_end - t1) - 1), rr.o_nx, rr.oe_nx);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    uint4 mw;
    uint32_t kr[KR];
    if constexpr (RG) {
#pragma unroll
        for (int i = 0; i < KR; ++i) kr[i] = 0u;
    }
    uint4 vr[16];
    const uint16_t* vbh = a.v + (size_t)bh * a.S_cap * 128;
    // a wave without a tile (or an empty block) reads row min(t0, S-1)
    const int tf0 = min(blk_begin + wave * DECODE_TILE, S - 1);
    const int ntf0 = max(1, min(DECODE_TILE, blk_end - tf0));
    if constexpr (RG) load_row_ragged(a, bh, tf0 + min(L, ntf0 - 1), o0, oe0, mw, kr, rr);
    else load_row<T>(a, bh, tf0, ntf0, L, mw, kr);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* lst = wbase + (size_t)wave * WAVE;
    float* ptab = reinterpret_cast<float*>(wbase + (size_t)wave * WAVE + LIST);
    if constexpr (RG) {
        // slots past a row read whatever entry they find: start every entry
        // at a valid table offset (channel 0)
        for (uint32_t i = (uint32_t)L; i < LIST / 16u; i += 64u) reinterpret_cast<uint4*>(lst)[i] = make_uint4(0, 0, 0, 0);
    }
    // the first tile's slot list needs only its masks: build it before
    // waiting for the table, then request the tile's V rows
    build_list<T>(mw, lst, L);
    __builtin_amdgcn_sched_barrier(0);
    load_v_tile(vbh, tf0, ntf0, L >> 4, L & 15, vr);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int j = tid + i * DECODE_FAST_THREADS;
        const float qv = bf16_to_f32(qb[i]) * a.qscale;
        reinterpret_cast<float*>(tab + (j & 127) * TAB)[j >> 7] = qv;
        if (SMODE) qn[(j & 127) * G + (j >> 7)] = qv * ns;     // ns belongs to channel tid & 127 == j & 127
    }
    if (tid < 128) reinterpret_cast<float*>(tab + 128 * TAB)[tid] = rv;
    __syncthreads();

    // q' . r per head
    float cq[G];
    {
        const float4 e0 = *reinterpret_cast<const float4*>(tab + L * TAB);
        const float4 e1 = *reinterpret_cast<const float4*>(tab + (L + 64) * TAB);
        const float r0 = reinterpret_cast<const float*>(tab + 128 * TAB)[L];
        const float r1 = reinterpret_cast<const float*>(tab + 128 * TAB)[L + 64];
        cq[0] = wave_sum_dpp(e0.x * r0 + e1.x * r1);
        cq[1] = wave_sum_dpp(e0.y * r0 + e1.y * r1);
        cq[2] = wave_sum_dpp(e0.z * r0 + e1.z * r1);
        cq[3] = wave_sum_dpp(e0.w * r0 + e1.w * r1);
    }

    float m_run[G], l_run[G];
    f32x4 accm[8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m_run[g] = -INFINITY;
        l_run[g] = 0.f;
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) accm[nb] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // the first tile's V rows were requested before the table set-up; later
    // tiles request theirs at the start of the tile
    if (wave < ntiles) {
        const int t0 = blk_begin + wave * DECODE_TILE;
        const int t1 = t0 + NW * DECODE_TILE, t2 = t1 + NW * DECODE_TILE;
        fast_tile<G, T, SMODE, false, true, RG>(a, bh, tab, lst, ptab, vbh, cq, t0, min(DECODE_TILE, blk_end - t0),
                                                t1 < blk_end ? min(DECODE_TILE, blk_end - t1) : 0, L, mw, kr, vr,
                                                m_run, l_run, accm, qn, rr,
                                                t2 < blk_end ? min(DECODE_TILE, blk_end - t2) : 0);
    }
    for (int tile = wave + NW; tile < ntiles; tile += NW) {
        const int t0 = blk_begin + tile * DECODE_TILE;
        const int t1 = t0 + NW * DECODE_TILE, t2 = t1 + NW * DECODE_TILE;   // this wave's next two tiles, if any
        uint4 vt[16];
        fast_tile<G, T, SMODE, true, false, RG>(a, bh, tab, lst, ptab, vbh, cq, t0, min(DECODE_TILE, blk_end - t0),
                                                t1 < blk_end ? min(DECODE_TILE, blk_end - t1) : 0, L, mw, kr, vt,
                                                m_run, l_run, accm, qn, rr,
                                                t2 < blk_end ? min(DECODE_TILE, blk_end - t2) : 0);
    }

    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) acc[g][nb] = accm[nb][g];
    finish_block<G, DECODE_FAST_THREADS, true>(a, m_run, l_run, acc, wbase,
                                               reinterpret_cast<int*>(smem + TABLES), bh, b, h, split);
}

// LDS bytes the fast kernel needs: tables and flag, then per wave the slot
// list and p, or the block / split merge scratch (reused after the tile
// loop). Must not exceed its static size: DECODE_FAST_LDS_BYTES, or
// DECODE_FAST_RAGGED_LDS_BYTES for ragged rows (T = 128).
uint32_t decode_fast_lds_bytes(int G, int T, int nsplit) {
    const uint32_t tab = 128u * 16u + 128u * 4u + 16u;   // q' float4 and r per channel, flag
    const uint32_t list = list_bytes_of(T);
    const uint32_t waves = DECODE_FAST_THREADS / 64;
    uint32_t dyn = waves * (list + 64u * (uint32_t)G * 4u);
    const uint32_t fin = finish_scratch_bytes(G, DECODE_FAST_THREADS, nsplit);
    if (fin > dyn) dyn = fin;
    return tab + dyn;
}

bool decode_fast_supported(int G, int T) { return G == 4 && (T == 26 || T == 38 || T == 48 || T == 64); }
// (the ragged rows' loads assume a region of at least 65 dwords: S >= 2)
bool decode_fast_ragged_supported(int G, int S) { return G == 4 && S >= 2; }


template <int SMODE, bool VP, bool RG>
hipError_t launch_generic(const DecodeArgs& a, int G, dim3 grid, dim3 block, hipStream_t stream) {
    const size_t lds = a.lay.lds_bytes;
    const void* fn = nullptr;
    switch (G) {
        case 1: fn = reinterpret_cast<const void*>(&decode_kernel<1, SMODE, VP, RG>); break;
        case 2: fn = reinterpret_cast<const void*>(&decode_kernel<2, SMODE, VP, RG>); break;
        case 4: fn = reinterpret_cast<const void*>(&decode_kernel<4, SMODE, VP, RG>); break;
        case 8: fn = reinterpret_cast<const void*>(&decode_kernel<8, SMODE, VP, RG>); break;
        default: return hipErrorInvalidValue;
    }
    if (lds > 65536) {
        // LDS above 64 KiB per workgroup must be requested explicitly (160 KiB per CU on gfx950)
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_kernel<1, SMODE, VP, RG>), grid, block, lds, stream, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<2, SMODE, VP, RG>), grid, block, lds, stream, a); break;
        case 4: hipLaunchKernelGGL((decode_kernel<4, SMODE, VP, RG>), grid, block, lds, stream, a); break;
        default: hipLaunchKernelGGL((decode_kernel<8, SMODE, VP, RG>), grid, block, lds, stream, a); break;
    }
    return hipGetLastError();
}

template <int SMODE>
hipError_t launch_fast(const DecodeArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
    switch (a.T) {
        case 26: hipLaunchKernelGGL((decode_fast_kernel<4, 26, SMODE>), grid, block, 0, stream, a); break;
        case 38: hipLaunchKernelGGL((decode_fast_kernel<4, 38, SMODE>), grid, block, 0, stream, a); break;
        case 48: hipLaunchKernelGGL((decode_fast_kernel<4, 48, SMODE>), grid, block, 0, stream, a); break;
        default: hipLaunchKernelGGL((decode_fast_kernel<4, 64, SMODE>), grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

// One launch: the split blocks, the last of which per (b, KV head) merges.
// G = 4 takes the matrix-core kernel for ragged rows (S >= 2), for the fixed
// T it is specialised for (fixed or sampled F), and the generic kernel
// otherwise; packed V always takes the generic kernel.
hipError_t launch_decode(const DecodeArgs& a, int G, int BH, hipStream_t stream) {
    const dim3 grid(a.nsplit, BH), block(DECODE_THREADS);
    if (a.row_off) {
        if (!decode_fast_ragged_supported(G, a.S)) return launch_generic<0, false, true>(a, G, grid, block, stream);
        if (decode_fast_lds_bytes(G, 128, a.nsplit) > (uint32_t)DECODE_FAST_RAGGED_LDS_BYTES) return hipErrorInvalidValue;
        hipLaunchKernelGGL((decode_fast_kernel<4, 128, 0, true>), grid, dim3(DECODE_FAST_THREADS), 0, stream, a);
        return hipGetLastError();
    }
    if (a.v_packed_mode) return launch_generic<0, true, false>(a, G, grid, block, stream);
    if (decode_fast_supported(G, a.T)) {
        const dim3 fblock(DECODE_FAST_THREADS);
        // the fast kernel's LDS is static (DECODE_FAST_LDS_BYTES)
        if (decode_fast_lds_bytes(G, a.T, a.nsplit) > (uint32_t)DECODE_FAST_LDS_BYTES) return hipErrorInvalidValue;
        switch (a.sampled) {
            case 0: return launch_fast<0>(a, grid, fblock, stream);
            case 4: return launch_fast<4>(a, grid, fblock, stream);
            case 5: return launch_fast<5>(a, grid, fblock, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (a.sampled) {
        case 0: return launch_generic<0, false, false>(a, G, grid, block, stream);
        case 4: return launch_generic<4, false, false>(a, G, grid, block, stream);
        case 5: return launch_generic<5, false, false>(a, G, grid, block, stream);
        default: return hipErrorInvalidValue;
    }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t value, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

}  // namespace spark
