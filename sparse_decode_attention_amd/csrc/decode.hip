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
#include "decode_common.h"
#include "decode_fast.h"

namespace spark {

namespace {

int tab_stride_for(int G) {
    switch (G) {
        case 1: return (int)sizeof(TabEntry<1>);
        case 2: return (int)sizeof(TabEntry<2>);
        case 4: return (int)sizeof(TabEntry<4>);
        default: return (int)sizeof(TabEntry<8>);
    }
}

}  // namespace

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

// SMODE: 0 for the recovery vector r, else the sampled F (4 Gaussian,
// 5 Exponential). Sampled F, G <= 4: two waves per SIMD (it fits without
// spills), so the Philox and sample arithmetic of one wave covers the
// latency of the other.
//
// VM 1: the V cache is packed too (V channels pruned): its rows and masks
// are loaded one tile ahead like the keys', staged in LDS, and expanded in
// P.V. VM 2: V pruned in 8-channel blocks, read straight into the P.V
// registers (load_v_tile_blocks), its tile's masks just before.
//
// RG: ragged packed rows (SparK-p): per-lane row starts and counts; the score
// loop runs to the wave's longest row, shorter rows pointing their surplus
// slots at a zero table entry and reading 0 for their values.
template <int G, int SMODE, int VM, bool RG>
__global__ void __launch_bounds__(DECODE_THREADS) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 2 : 1)))
decode_kernel(const DecodeArgs a) {
    constexpr bool SAMPLED = SMODE != 0;
    constexpr bool VP = VM == 1;
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

    const uint16_t* vbh = VP ? nullptr
                             : VM == 2 ? a.v_packed + (size_t)bh * a.S_cap * a.nbv * 8 : a.v + (size_t)bh * a.S_cap * 128;
    const uint16_t* vmh = VM == 2 ? a.v_bmask + (size_t)bh * vblock_mask_stride(a.S_cap) : nullptr;
    uint4 rvo = make_uint4(0, 0, 0, 0);     // VM 2: this lane's recovery block in bf16
    if (VM == 2) {
        const float4* rq = reinterpret_cast<const float4*>(a.rv + (size_t)bh * 128 + 8 * oct);
        rvo = vblock_recovery(rq[0], rq[1]);
    }
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
        if (VM == 0) load_v_tile(vbh, t0, nt, tau, oct, vr);
        uint32_t vkept = 0u;    // VM 2: which of vr hold kept blocks
        if (VM == 2) {
            uint4 vm[2];
            load_vblock_masks(vmh, t0, tau, vm);
            vkept = load_v_tile_blocks(vbh, vm, a.nbv, t0, nt, tau, oct, vr);
        }
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
        else {
            if (VM == 2) vblock_fill(vr, vkept, rvo);
            pv_tile<G>(vr, ptab, acc, tau);
        }
        wave_lds_sync();
    }

    __shared__ int s_last;
    finish_block<G, DECODE_THREADS, false>(a, m_run, l_run, acc, wbase, &s_last, bh, b, h, split);
}

// the exact-T variants: G = 4 at T in {26, 38, 48, 64} with every F, at the
// other tenths of lambda with the fixed F, and G = 1, 2, 8 at T in {26, 64}
bool decode_fast_exact(int G, int T, int sampled) {
    const bool base = G == 4 && (T == 26 || T == 38 || T == 48 || T == 64);
    if (sampled) return base;
    if (G == 4) return base || T == 13 || T == 51 || T == 77 || T == 90 || T == 102 || T == 115;
    return (G == 1 || G == 2 || G == 8) && (T == 26 || T == 64);
}

bool decode_fast_supported(int G, int T, int sampled, size_t packed_elems) {
    if (G != 1 && G != 2 && G != 4 && G != 8) return false;
    if (sampled) return decode_fast_exact(G, T, sampled);
    if (T < 1 || T > 128) return false;
    // rows that are not exact 16-byte multiples: each lane's 16-byte requests
    // start inside the packed buffer and must fit in it when they start at
    // its first dword
    const int kr = decode_fast_exact(G, T, 0) ? decode_fast_kr_exact(T) : decode_fast_kr(decode_fast_bucket(T), (T & 1) != 0);
    return T % 2 == 0 && decode_fast_exact(G, T, 0) ? true : packed_elems / 2 >= (size_t)kr;
}
// (the ragged rows' loads assume a region of at least 65 dwords: S >= 2)
bool decode_fast_ragged_supported(int G, int S) { return (G == 1 || G == 2 || G == 4 || G == 8) && S >= 2; }

template <int SMODE, int VM, bool RG>
hipError_t launch_generic(const DecodeArgs& a, int G, dim3 grid, dim3 block, hipStream_t stream) {
    const size_t lds = a.lay.lds_bytes;
    const void* fn = nullptr;
    switch (G) {
        case 1: fn = reinterpret_cast<const void*>(&decode_kernel<1, SMODE, VM, RG>); break;
        case 2: fn = reinterpret_cast<const void*>(&decode_kernel<2, SMODE, VM, RG>); break;
        case 4: fn = reinterpret_cast<const void*>(&decode_kernel<4, SMODE, VM, RG>); break;
        case 8: fn = reinterpret_cast<const void*>(&decode_kernel<8, SMODE, VM, RG>); break;
        default: return hipErrorInvalidValue;
    }
    if (lds > 65536) {
        // LDS above 64 KiB per workgroup must be requested explicitly (160 KiB per CU on gfx950)
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_kernel<1, SMODE, VM, RG>), grid, block, lds, stream, a); break;
        case 2: hipLaunchKernelGGL((decode_kernel<2, SMODE, VM, RG>), grid, block, lds, stream, a); break;
        case 4: hipLaunchKernelGGL((decode_kernel<4, SMODE, VM, RG>), grid, block, lds, stream, a); break;
        default: hipLaunchKernelGGL((decode_kernel<8, SMODE, VM, RG>), grid, block, lds, stream, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_fast_g(const DecodeArgs& a, int G, dim3 grid, hipStream_t stream) {
    switch (G) {
        case 1: return launch_fast_g1(a, grid, stream);
        case 2: return launch_fast_g2(a, grid, stream);
        case 4: return launch_fast_g4(a, grid, stream);
        case 8: return launch_fast_g8(a, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

// One launch: the split blocks, the last of which per (b, KV head) merges.
// The matrix-core kernel takes ragged rows (S >= 2) and, for fixed or
// sampled F, the shapes decode_fast_supported admits (an exact-T variant
// where one exists, else the runtime-T variant of T's bucket); packed V and
// everything else take the generic kernel.
hipError_t launch_decode(const DecodeArgs& a, int G, int BH, hipStream_t stream) {
    const dim3 grid(a.nsplit, BH), block(DECODE_THREADS);
    if (a.row_off) {
        if (!decode_fast_ragged_supported(G, a.S)) return launch_generic<0, 0, true>(a, G, grid, block, stream);
        return launch_fast_g(a, G, grid, stream);
    }
    if (a.v_packed_mode == 1) return launch_generic<0, 1, false>(a, G, grid, block, stream);
    if (a.v_packed_mode == 2) {
        if (!decode_fast_supported(G, a.T, 0, a.packed_elems)) return launch_generic<0, 2, false>(a, G, grid, block, stream);
        switch (G) {
            case 1: return launch_fast_vb_g1(a, grid, stream);
            case 2: return launch_fast_vb_g2(a, grid, stream);
            case 4: return launch_fast_vb_g4(a, grid, stream);
            case 8: return launch_fast_vb_g8(a, grid, stream);
            default: return hipErrorInvalidValue;
        }
    }
    if (decode_fast_supported(G, a.T, a.sampled, a.packed_elems)) {
        if (G == 4 && (a.T == 26 || a.T == 38 || a.T == 48 || a.T == 64)) return launch_fast_fixed(a, grid, stream);
        if (decode_fast_exact(G, a.T, a.sampled)) return launch_fast_fixed2(a, G, grid, stream);
        return launch_fast_g(a, G, grid, stream);
    }
    switch (a.sampled) {
        case 0: return launch_generic<0, 0, false>(a, G, grid, block, stream);
        case 4: return launch_generic<4, 0, false>(a, G, grid, block, stream);
        case 5: return launch_generic<5, 0, false>(a, G, grid, block, stream);
        default: return hipErrorInvalidValue;
    }
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t value, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

}  // namespace spark
