// Matrix-core decode kernel (internal header; instantiated per group size in
// decode_fast_g*.hip). Same arithmetic as the generic kernel (walkthrough
// section 3.3, decode half of Fig. 3): the sparse-form score
//     q'_g . k_hat_t = q'_g . r + sum over kept j of q'_g,j (k_tj - r_j),
// online softmax in base 2, then P.V over the dense V, but with
//   - 8 waves per block, one block per CU;
//   - each lane's packed row loaded straight into registers (no LDS staging),
//     so a slot's register is known at compile time: the score loop is
//     unrolled for the largest row of the variant, and runs to the row length
//     T with a wave-uniform exit;
//   - the slot list of a tile as u16 table offsets, lane-major in LDS;
//   - P.V on the matrix cores (v_mfma_f32_16x16x16_bf16) with p split into
//     a bf16 hi and lo part, V taken from the registers it was loaded into.
//
// Variants (template parameters):
//   TFIX > 0  exact row length TFIX (the pruning ratios in common use): the
//             slot loop runs exactly T slots;
//   TB        otherwise: any T with T <= TB (buckets 32, 64, 96, 128), the
//             slot loop unrolled for TB with a wave-uniform exit at T;
//   ODD       odd T: rows start mid-dword on every other token and are
//             realigned with a funnel shift.
//   Rows of an even exact T are read exactly (16-byte loads when T is a
//   multiple of 8, single dwords otherwise); every other row as 16-byte
//   loads from the dword holding its first element;
//   RG        ragged rows (SparK-p): per-lane row offsets and lengths;
//   SMODE     sampled recovery F (4 Gaussian, 5 Exponential), TFIX only;
//   VB        V pruned in 8-channel blocks: each lane's 16-byte V block read
//             from its slot in the packed V row, or the recovery block.
#pragma once
#include "decode_common.h"

namespace spark {

namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int FAST_NW = DECODE_FAST_THREADS / 64;

// Two fp32 -> packed bf16 pair (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Slot of token t (0..63) in a ptab row: within each 16-token group the
// token 16 grp + 4 e + tau sits at 16 grp + 4 tau + e, so the four tokens
// that one lane of the matrix-core P.V needs are adjacent.
__device__ __forceinline__ uint32_t ptab_slot(uint32_t t) { return (t & 48u) | ((t & 3u) << 2) | ((t >> 2) & 3u); }

// ---- q' and r tables in LDS, 16 bytes per channel: channel c's q' of heads
// 0-3 (min(G, 4) fp32) at byte 16 c, heads 4-7 of G = 8 in a second table
// 2 KiB further on, r at byte 16 c of the table after those. A slot-list
// entry is u = 16 c, so one address register serves every read of a slot
// (the table distances go into the LDS instructions' offset fields).
__host__ __device__ constexpr uint32_t fast_rtab(int G) { return G == 8 ? 4096u : 2048u; }
__host__ __device__ constexpr uint32_t fast_tables_bytes(int G) { return fast_rtab(G) + 2048u; }
template <int G>
__device__ __forceinline__ uint32_t qtab_offset(uint32_t c, uint32_t g) {
    return (g >> 2) * 2048u + c * 16u + (g & 3u) * 4u;
}

template <int G>
struct QV { float v[G]; };
template <int G>
__device__ __forceinline__ QV<G> load_qrow(const unsigned char* tab, uint32_t u) {
    QV<G> r;
    if constexpr (G == 1) {
        r.v[0] = *reinterpret_cast<const float*>(tab + u);
    } else if constexpr (G == 2) {
        const float2 x = *reinterpret_cast<const float2*>(__builtin_assume_aligned(tab + u, 16));
        r.v[0] = x.x; r.v[1] = x.y;
    } else {
        const float4 x = *reinterpret_cast<const float4*>(__builtin_assume_aligned(tab + u, 16));
        r.v[0] = x.x; r.v[1] = x.y; r.v[2] = x.z; r.v[3] = x.w;
        if constexpr (G == 8) {
            const float4 y = *reinterpret_cast<const float4*>(__builtin_assume_aligned(tab + u + 2048u, 16));
            r.v[4] = y.x; r.v[5] = y.y; r.v[6] = y.z; r.v[7] = y.w;
        }
    }
    return r;
}

// ---- matrix-core softmax and P.V. The 16 x 16 A operand of a P.V MFMA has
// one row per (head, part): row m < G is bf16(p) of head m, row G <= m < 2G
// is the remainder p - bf16(p) of head m - G (together p to about 2^-16),
// rows from 2G on are zero. Output tile D: lane l holds rows 4 (l >> 4) + e,
// e = 0..3, of column l & 15; alpha of row m is that of head m mod G.
template <int G>
__device__ __forceinline__ f32x4 row_alpha(const float (&al)[G], int L) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
    if constexpr (G == 1) return (f32x4){al[0], al[0], al[0], al[0]};
    else if constexpr (G == 2) return (f32x4){al[0], al[1], al[0], al[1]};
    else if constexpr (G == 4) return (f32x4){al[0], al[1], al[2], al[3]};
    else {
        // rows 4 (l >> 4) + e: heads e (lanes 0-15, 32-47) or 4 + e (16-31,
        // 48-63); a select of whole vectors (selecting array elements makes
        // the compiler index a scratch copy of the array)
        const f32x4 lo = {al[0], al[1], al[2], al[3]}, hi = {al[4], al[5], al[6], al[7]};
        return ((L >> 4) & 1) != 0 ? hi : lo;
    }
}

// Online softmax of one tile: p goes to ptab as [g][64 token slots] fp32;
// the accumulator rows are rescaled by their head's alpha.
template <int G>
__device__ __forceinline__ void softmax_tile_mf(const float (&s)[G], float (&m_run)[G], float (&l_run)[G],
                                                f32x4 (&accm)[8], float* ptab, int L) {
    float al[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mt = wave_max_dpp(s[g]);
        const float mn = fmaxf(m_run[g], mt);
        // hardware exp2 (v_exp_f32, about 1 ulp, no denormal rescaling):
        // both arguments are <= 0, so every value is at most 1
        al[g] = __builtin_amdgcn_exp2f(m_run[g] - mn);
        const float p = __builtin_amdgcn_exp2f(s[g] - mn);
        l_run[g] = l_run[g] * al[g] + p;
        m_run[g] = mn;
        ptab[g * 64 + ptab_slot((uint32_t)L)] = p;
    }
    const f32x4 alpha = row_alpha<G>(al, L);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) accm[nb] *= alpha;
}

// P.V of one 64-token tile, V from the registers it was loaded into: lane
// (tau, oct) holds vr[i] = V row 4i + tau, d in [8 oct, 8 oct + 8). Per
// 16-token group grp and column offset j (0..7), with K index k = 4 tau + e
// standing for token 16 grp + 4 e + tau:
//   A: the rows above, lane l supplying row l & 15 for k in 4 (l >> 4) + 0..3;
//   B (16 x 16): B[k][n] = V[token(k)][8 n + j], element j of
//                vr[4 grp + e] in lane (tau, n), two byte permutes per MFMA;
//   D: accm[j], column n = d = 8 n + j.
// No V bytes go through LDS.
__device__ __forceinline__ uint32_t dword_of(const uint4& x, int j) {
    return j == 0 ? x.x : j == 1 ? x.y : j == 2 ? x.z : x.w;
}
template <int G>
__device__ __forceinline__ void pv_tile_mf(const uint4 (&vr)[16], const float* ptab, f32x4 (&accm)[8], int L) {
    const uint32_t m = (uint32_t)L & 15u, q = (uint32_t)L >> 4;
    const uint32_t hg = m & (uint32_t)(G - 1);
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
        const float4 pv = *reinterpret_cast<const float4*>(ptab + hg * 64u + 16u * grp + 4u * q);
        const uint32_t hi0 = pack_bf16(pv.x, pv.y), hi1 = pack_bf16(pv.z, pv.w);
        const uint32_t lo0 = pack_bf16(pv.x - bf16_lo(hi0), pv.y - bf16_hi(hi0));
        const uint32_t lo1 = pack_bf16(pv.z - bf16_lo(hi1), pv.w - bf16_hi(hi1));
        const u32x2 aw = {m < (uint32_t)G ? hi0 : (m < 2u * G ? lo0 : 0u),
                          m < (uint32_t)G ? hi1 : (m < 2u * G ? lo1 : 0u)};
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

// Add the hi and lo rows of each head: lanes 0-15 end with acc[g][j] of
// d = 8 (lane & 15) + j (the layout the block merge takes).
template <int G>
__device__ __forceinline__ void combine_mf(const f32x4 (&accm)[8], float (&acc)[G][8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if constexpr (G == 1) {
            acc[0][j] = accm[j][0] + accm[j][1];
        } else if constexpr (G == 2) {
            acc[0][j] = accm[j][0] + accm[j][2];
            acc[1][j] = accm[j][1] + accm[j][3];
        } else if constexpr (G == 4) {
#pragma unroll
            for (int g = 0; g < 4; ++g) acc[g][j] = xor16_sum(accm[j][g]);   // hi rows (lanes 0-15) + lo rows (16-31)
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // hi rows in lanes 0-31, lo rows in 32-63; heads 4-7 then move from lanes 16-31 to 0-15
                const float y = xor32_sum(accm[j][e]);
                acc[e][j] = y;
                acc[4 + e][j] = __shfl_xor(y, 16, 64);
            }
        }
    }
}

// ---- packed rows into registers. Lanes past the end of a partial tile
// re-read the last valid row (their scores are discarded).
struct RowState {
    int sh, c;        // element shift of the row within its first dword; ragged rows: its length
    int o_nx, oe_nx;  // ragged rows: offsets of the next tile's row (requested a tile ahead)
};

// Exact rows of a compile-time even T: T / 16 16-byte loads per lane when
// T is a multiple of 8 (rows 16-byte aligned), else T / 2 dword loads (rows
// 4-byte aligned; measured faster here than 16-byte loads at 4-byte
// alignment: T = 26: 22.6 against 24.5 us at S = 32K).
template <int T>
__device__ __forceinline__ void load_row_fixed(const DecodeArgs& a, int bh, int t0, int nt, int L,
                                               uint4& mw, uint32_t (&kr)[T / 2]) {
    static_assert(T % 2 == 0, "even rows");
    const size_t row = (size_t)bh * a.S_cap + t0 + min(L, nt - 1);
    mw = *reinterpret_cast<const uint4*>(a.mask + row * 4);
    if constexpr (T % 8 == 0) {
        const uint4* src = reinterpret_cast<const uint4*>(a.packed + row * T);
#pragma unroll
        for (int i = 0; i < T / 8; ++i) {
            const uint4 x = src[i];
            kr[4 * i] = x.x; kr[4 * i + 1] = x.y; kr[4 * i + 2] = x.z; kr[4 * i + 3] = x.w;
        }
    } else {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(a.packed + row * T);
#pragma unroll
        for (int i = 0; i < T / 2; ++i) kr[i] = src[i];
    }
}

// Rows of any other T (a runtime T <= TB, or an exact T that is not a
// multiple of 8): the lane requests KR dwords (KR / 4 16-byte
// requests, no branches) from the one holding its row's first element, so
// kr[i] holds slots 2 i - sh and 2 i - sh + 1 (sh = 1 when the row starts in
// the middle of a dword: odd T only). What lies past the row belongs to the
// next rows and is never used. A lane whose KR dwords would leave the packed
// buffer (the last rows of the buffer) requests the buffer's first KR
// instead and then, in a branch taken only when the wave has such a lane,
// its own row's dwords one by one, the buffer's last element on its own
// when it ends mid-dword.
template <int KR, bool ODD>
__device__ __forceinline__ void load_row_rt(const DecodeArgs& a, int T, int bh, int t0, int nt, int L, uint4& mw,
                                            uint32_t (&kr)[KR], RowState& rs) {
    static_assert(KR % 4 == 0, "whole 16-byte requests");
    typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
    // wave-uniform: the tile's first row, its first element, the dword
    // holding it, and the whole dwords from there to the buffer's end
    const size_t row0 = (size_t)bh * a.S_cap + t0;
    const size_t o0 = row0 * (size_t)T;
    const uint32_t* base = reinterpret_cast<const uint32_t*>(a.packed);
    const uint32_t* wbase = base + (o0 >> 1);
    const size_t e_dw = a.packed_elems >> 1;
    const uint32_t room = (uint32_t)min(e_dw - (o0 >> 1), (size_t)0x40000000u);
    // per lane, 32-bit: its row's first element and dword from wbase
    const uint32_t l = (uint32_t)min(L, nt - 1);
    mw = *reinterpret_cast<const uint4*>(a.mask + row0 * 4 + l * 4u);
    const uint32_t le = l * (uint32_t)T + (uint32_t)(o0 & 1);
    const uint32_t ldw = le >> 1;
    rs.sh = ODD ? (int)(le & 1u) : 0;
    const bool near_end = ldw + (uint32_t)KR > room;
    const uint32_t* src = near_end ? base : wbase + ldw;
#pragma unroll
    for (int i = 0; i < KR / 4; ++i) {
        const u32x4_a4 x = *reinterpret_cast<const u32x4_a4*>(src + 4 * i);
        kr[4 * i] = x.x; kr[4 * i + 1] = x.y; kr[4 * i + 2] = x.z; kr[4 * i + 3] = x.w;
    }
    if (ballot(near_end) != 0) {
        if (near_end) {
            const int ndw = ((int)(le & 1u) + T + 1) >> 1;
            const size_t o_dw = (o0 >> 1) + ldw;
            // the buffer's last element, when it ends mid-dword
            const uint32_t last = (a.packed_elems & 1) != 0 ? (uint32_t)a.packed[a.packed_elems - 1] : 0u;
            // whole dwords from the row's first to the buffer's end (0 when a
            // one-element row is the buffer's last, odd, element)
            const uint32_t n_in = (uint32_t)(e_dw - min(o_dw, e_dw));
#pragma unroll
            for (int i = 0; i < KR; ++i) {
                const uint32_t x = base[min(o_dw + (size_t)i, e_dw - 1)];   // (e_dw >= KR, checked on the host)
                if (i < ndw) kr[i] = (uint32_t)i < n_in ? x : last;
            }
        }
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
__device__ __forceinline__ void ragged_offsets(const DecodeArgs& a, int bh, int t, int& o, int& oe) {
    const int32_t* ro = a.row_off + (size_t)bh * (a.S + 1);
    o = ro[t];
    oe = ro[t + 1];
}
__device__ __forceinline__ void load_row_ragged(const DecodeArgs& a, int bh, int t, int o, int oe, uint4& mw,
                                                uint32_t (&kr)[RAGGED_KR], RowState& rr) {
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

// ---- slot list. Row stride (u16 elements) of the lane-major list: room for
// T slots and a spare one, rounded up to a multiple of 4 so that every row
// starts 8-byte aligned (the list writes combine into 8-byte stores).
__host__ __device__ constexpr uint32_t list_stride_of(int T) { return ((uint32_t)T + 5u) & ~3u; }
// LDS bytes of one wave's slot list, in whole 16-byte units
__host__ __device__ constexpr uint32_t list_bytes_of(int T) { return (64u * list_stride_of(T) * 2u + 15u) & ~15u; }
// the list of a runtime T <= TB: the stride of any such T, and 16 spare
// entries after the last lane's row (the score loop reads up to 2 NB - 2 <= 14
// entries past a row, which it never uses: the next lane's, or these)
__host__ __device__ constexpr uint32_t list_bytes_rt(int TB) {
    return ((64u * ((uint32_t)TB + 4u) + 16u) * 2u + 15u) & ~15u;
}

// Slot list of one tile, lane-major: lst[lane * stride + rho] = 16 c for the
// lane's rho-th kept channel c (ascending). One bit-clearing loop per mask
// word; lanes leave it as their word empties.
__device__ __forceinline__ void build_list(const uint4& mw, uint8_t* lst, int L, uint32_t stride) {
    uint16_t* p = reinterpret_cast<uint16_t*>(lst) + (uint32_t)L * stride;
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
                p[i + u] = (uint16_t)(((uint32_t)__builtin_ctz(m) << 4) | (512u * w));
                m &= m - 1;
            }
        }
        for (; i < pc; ++i) {
            p[i] = (uint16_t)(((uint32_t)__builtin_ctz(m) << 4) | (512u * w));
            m &= m - 1;
        }
        p += pc;
    }
}

// Compile-time shape of a variant.
template <int G, int TB, int TFIX, bool ODD, bool RG>
struct FastCfg {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
    static_assert(RG ? (TFIX == 0 && TB == 128) : TFIX ? (TB == TFIX && ODD == ((TFIX & 1) != 0) && TFIX < 128)
                                                       : (TB == 32 || TB == 64 || TB == 96 || TB == 128),
                  "variant");
    // exact rows of an even length: loaded exactly (load_row_fixed)
    static constexpr bool XLOAD = TFIX != 0 && TFIX % 2 == 0;
    // slots the score loop is unrolled for
    static constexpr int LOOP = RG ? 128 : TB;
    // row registers per lane
    static constexpr int KR = RG ? RAGGED_KR : TFIX ? decode_fast_kr_exact(TFIX) : decode_fast_kr(TB, ODD);
    // slots per batch of the score loop (4 where the row registers or the
    // q' rows of eight heads would otherwise crowd out the rest)
    static constexpr int NB = (G == 8 || RG || KR > 40) ? 4 : 8;
    // the smallest row length the variant serves (the previous bucket's
    // largest plus one): batches below it are always full
    static constexpr int TMIN = RG ? 0 : TFIX ? TFIX : (TB == 32 ? 1 : TB - 31);
    static constexpr uint32_t LIST = RG ? list_bytes_of(128) : TFIX ? list_bytes_of(TFIX) : list_bytes_rt(TB);
    static constexpr uint32_t WAVE = LIST + 64u * (uint32_t)G * 4u;
    // static LDS: the tables and a 16-byte flag slot, then the waves'
    // regions (the exact-T variants keep the size of the largest of them,
    // 64); at least 72 KiB, so that any u16 list entry (even one a mask with
    // fewer than T bits left unwritten) addresses LDS inside the block's
    static constexpr uint32_t LDS_NEED = fast_tables_bytes(G) + 16u + (uint32_t)FAST_NW * WAVE;
    static constexpr uint32_t LDS = (TFIX && LDS_NEED <= DECODE_FAST_LDS_BYTES) ? DECODE_FAST_LDS_BYTES
                                                                                : (LDS_NEED > 73728u ? LDS_NEED : 73728u);
    static_assert(LDS_NEED <= LDS && 65535u + fast_rtab(G) + 4u <= LDS, "LDS");
};

// Block-pruned V (VB): the head's block masks, the tile's masks of this
// lane's rows (requested one tile ahead, before the tile's packed rows) and
// this lane's recovery block in bf16.
struct VBlockState {
    const uint16_t* vmh = nullptr;
    uint4 vm[2] = {};
    uint4 rvo = {};
    uint32_t kbits = 0u;     // which V registers of the tile hold kept blocks
};

// One 64-token tile. The slot list is built from the tile's mask (before the
// call when LIST_READY); then the tile's V rows are requested (unless LOAD_V
// is false: then the prologue did), so they arrive during the score loop and
// the softmax; the next tile's mask and packed rows are requested once the
// scores have consumed this tile's; then P.V. A request made while the memory
// queue is full stalls the wave, so none is placed ahead of work that needs
// no memory.
//
// Score loop: slots in batches of NB, the batch's list entries requested one
// batch ahead so that their LDS round trip overlaps the previous batch's
// gathers. Exact T: every batch full. Runtime T: batches up to T, the slots
// of the last one past T adding nothing (their list entries are valid
// offsets, their values are replaced by 0). Ragged rows: batches up to the
// wave's longest row, each slot past its lane's row adding nothing (its
// list entry is a stale but valid table offset, its value is discarded).
template <int G, int TB, int TFIX, bool ODD, int SMODE, bool LOAD_V, bool LIST_READY, bool RG, bool VB>
__device__ __forceinline__ void fast_tile(const DecodeArgs& a, int T, uint32_t lstride, int bh,
                                          const unsigned char* tab, uint8_t* lst, float* ptab, const uint16_t* vbh,
                                          const float (&cq)[G], int t0, int nt, int nt_next, int L, uint4& mw,
                                          uint32_t (&kr)[FastCfg<G, TB, TFIX, ODD, RG>::KR], uint4 (&vr)[16],
                                          float (&m_run)[G], float (&l_run)[G], f32x4 (&accm)[8], const float* qn,
                                          RowState& rs, int nt_next2, VBlockState& vbs) {
    using C = FastCfg<G, TB, TFIX, ODD, RG>;
    constexpr int NB = C::NB, LOOP = C::LOOP;
    const int tau = L >> 4, oct = L & 15;
    const int t1 = t0 + FAST_NW * DECODE_TILE;
    if constexpr (!LIST_READY) build_list(mw, lst, L, lstride);
    if constexpr (LOAD_V) {
        if constexpr (VB) vbs.kbits = load_v_tile_blocks(vbh, vbs.vm, a.nbv, t0, nt, tau, oct, vr);
        else load_v_tile(vbh, t0, nt, tau, oct, vr);
    }
    wave_lds_sync();
    const uint16_t* lrow16 = reinterpret_cast<const uint16_t*>(lst) + (uint32_t)L * lstride;
    const unsigned char* rtab = tab + fast_rtab(G);
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s[g] = cq[g];
    // slots to score: T, or (ragged rows) the wave's longest row, wave-uniform
    const int nmax = RG ? (int)wave_max_dpp((float)rs.c) : T;
    const uint32_t sh16 = (RG || ODD) ? 16u * (uint32_t)rs.sh : 0u;
    uint32_t off_next[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k)
        if (k < LOOP) off_next[k] = lrow16[k];
    auto batch = [&](const int r0) __attribute__((always_inline)) {
        // keep each batch's loads inside the batch: unbounded hoisting across
        // the fully unrolled slot loop would need registers for every slot
        __builtin_amdgcn_sched_barrier(0);
        uint32_t off[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) off[k] = off_next[k];
        // (runtime T: the next batch's entries are read even past T, from
        // the next lane's row or the list's spare entries: unconditional
        // reads let the compiler rotate registers instead of copying them)
#pragma unroll
        for (int k = 0; k < NB; ++k)
            if (r0 + NB + k < LOOP) off_next[k] = lrow16[r0 + NB + k];
        QV<G> qv[NB];
        float rv[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (r0 + k < LOOP) {
                qv[k] = load_qrow<G>(tab, off[k]);
                rv[k] = *reinterpret_cast<const float*>(rtab + off[k]);
            }
        }
        float e[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (r0 + k < LOOP) {
                const int rho = r0 + k;
                uint32_t w;
                if constexpr (RG || ODD) w = __builtin_amdgcn_alignbit(kr[(rho >> 1) + 1], kr[rho >> 1], sh16);
                else w = kr[rho >> 1];
                const float kv = (rho & 1) ? bf16_hi(w) : bf16_lo(w);
                e[k] = kv - rv[k];
                if constexpr (RG) e[k] = rho < rs.c ? e[k] : 0.0f;
            }
        }
        if constexpr (TFIX == 0 && !RG) {
            // runtime T: only the last batch has slots past T; it clears them
            // in a branch of its own (the empty asm keeps the compiler from
            // turning the branch into selects that every batch would pay)
            if (r0 + NB > C::TMIN && r0 + NB > nmax) {
                asm volatile("");
#pragma unroll
                for (int k = 0; k < NB; ++k) e[k] = r0 + k < nmax ? e[k] : 0.0f;
            }
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (r0 + k < LOOP) {
#pragma unroll
                for (int g = 0; g < G; ++g) s[g] = fmaf(qv[k].v[g], e[k], s[g]);
            }
        }
        // consume the partial sums here: otherwise the compiler sinks the
        // FMAs of every batch to the end and keeps all gathered rows live
#pragma unroll
        for (int g = 0; g < G; ++g) asm volatile("" : "+v"(s[g]));
    };
    // (batches past the last are skipped one by one, uniformly: a loop with
    // an early exit would not be unrolled; batches that every T of the
    // variant fills need no test)
#pragma unroll
    for (int r0 = 0; r0 < LOOP; r0 += NB) {
        if (r0 + NB <= C::TMIN || r0 < nmax) batch(r0);
    }
    // sampled F: the sample term needs this tile's mask, so it runs before
    // the next tile's masks are requested into mw
    if constexpr (SMODE != 0) sampled_scores<G, SMODE == 4>(a, qn, mw, bh, t0, nt, L, s);
    if (L >= nt) {
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = -INFINITY;
    }
    // the packed rows are consumed: request the next tile's into them
    if constexpr (RG) {
        if (nt_next > 0) {
            load_row_ragged(a, bh, t1 + min(L, nt_next - 1), rs.o_nx, rs.oe_nx, mw, kr, rs);
            if (nt_next2 > 0)
                ragged_offsets(a, bh, t1 + FAST_NW * DECODE_TILE + min(L, nt_next2 - 1), rs.o_nx, rs.oe_nx);
        }
    } else {
        // block-pruned V: the next tile's block masks go first, so that
        // waiting for them does not wait for its packed rows
        if constexpr (VB) {
            if (nt_next > 0) load_vblock_masks(vbs.vmh, t1, tau, vbs.vm);
        }
        if constexpr (C::XLOAD) {
            if (nt_next > 0) load_row_fixed<TFIX>(a, bh, t1, nt_next, L, mw, kr);
        } else {
            if (nt_next > 0) load_row_rt<C::KR, ODD>(a, T, bh, t1, nt_next, L, mw, kr, rs);
        }
    }
    softmax_tile_mf<G>(s, m_run, l_run, accm, ptab, L);
    wave_lds_sync();
    if constexpr (VB) vblock_fill(vr, vbs.kbits, vbs.rvo);
    pv_tile_mf<G>(vr, ptab, accm, L);
    wave_lds_sync();
}

// Decode block: DECODE_FAST_THREADS threads (8 waves), one block per CU.
// Each lane loads its token's packed row straight into registers and builds
// the list of its kept channels in LDS as u16 table offsets; the score loop
// then knows each slot's register at compile time.
//
// SMODE 4 / 5: the sampled F (Gaussian / Exponential); the r table then holds
// mu / a_j, and a q' ns table of 128 G fp32 follows the other LDS.
template <int G, int TB, int TFIX, bool ODD, int SMODE, bool RG, bool VB>
__global__ void __launch_bounds__(DECODE_FAST_THREADS)
decode_fast_kernel(const DecodeArgs a) {
    using C = FastCfg<G, TB, TFIX, ODD, RG>;
    static_assert(SMODE == 0 || TFIX != 0, "sampled F on the exact-T variants only");
    static_assert(!VB || (SMODE == 0 && !RG), "block-pruned V with fixed rows and the fixed F");
    // statically sized LDS: its base address is a compile-time constant, so
    // table offsets fold into the LDS instructions' offset fields
    __shared__ __align__(16) unsigned char smem[C::LDS + (SMODE ? 128 * G * 4 : 0)];
    float* qn = reinterpret_cast<float*>(smem + C::LDS);   // [128][G], sampled F only
    constexpr uint32_t TABLES = fast_tables_bytes(G);       // then a 16-byte flag slot
    constexpr uint32_t LIST = C::LIST, WAVE = C::WAVE;
    constexpr int KR = C::KR;
    unsigned char* tab = smem;
    unsigned char* wbase = smem + TABLES + 16;
    const int T = TFIX ? TFIX : a.T;
    const uint32_t lstride = RG ? list_stride_of(128) : TFIX ? list_stride_of(TFIX) : list_stride_of(a.T);

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
    constexpr int QPT = (128 * G + DECODE_FAST_THREADS - 1) / DECODE_FAST_THREADS;
    uint16_t qb[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int j = tid + i * DECODE_FAST_THREADS;
        qb[i] = 0;
        if (j < 128 * G) qb[i] = a.q[((size_t)b * a.N_q + (size_t)h * G + (j >> 7)) * 128 + (j & 127)];
    }
    float rv = a.r[(size_t)bh * 128 + (tid & 127)];
    VBlockState vbs{};
    float4 rvq[2];       // block-pruned V: this lane's recovery block, converted once it has arrived
    if constexpr (VB) {
        const float4* rq = reinterpret_cast<const float4*>(a.rv + (size_t)bh * 128 + 8 * (L & 15));
        rvq[0] = rq[0];
        rvq[1] = rq[1];
    }
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
    RowState rs{};
    int o0 = 0, oe0 = 0;
    if constexpr (RG) {
        const int tr0 = min(blk_begin + wave * DECODE_TILE, S - 1);
        ragged_offsets(a, bh, tr0 + min(L, max(1, min(DECODE_TILE, blk_end - tr0)) - 1), o0, oe0);
        const int t1 = blk_begin + (wave + FAST_NW) * DECODE_TILE;
        if (t1 < blk_end) ragged_offsets(a, bh, t1 + min(L, min(DECODE_TILE, blk_end - t1) - 1), rs.o_nx, rs.oe_nx);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    uint4 mw;
    uint32_t kr[KR];
    if constexpr (TFIX == 0) {
#pragma unroll
        for (int i = 0; i < KR; ++i) kr[i] = 0u;
    }
    uint4 vr[16];
    const uint16_t* vbh = VB ? a.v_packed + (size_t)bh * a.S_cap * a.nbv * 8 : a.v + (size_t)bh * a.S_cap * 128;
    // a wave without a tile (or an empty block) reads row min(t0, S-1)
    const int tf0 = min(blk_begin + wave * DECODE_TILE, S - 1);
    const int ntf0 = max(1, min(DECODE_TILE, blk_end - tf0));
    if constexpr (VB) {
        vbs.vmh = a.v_bmask + (size_t)bh * vblock_mask_stride(a.S_cap);
        load_vblock_masks(vbs.vmh, tf0, L >> 4, vbs.vm);
    }
    if constexpr (RG) load_row_ragged(a, bh, tf0 + min(L, ntf0 - 1), o0, oe0, mw, kr, rs);
    else if constexpr (C::XLOAD) load_row_fixed<TFIX>(a, bh, tf0, ntf0, L, mw, kr);
    else load_row_rt<KR, ODD>(a, T, bh, tf0, ntf0, L, mw, kr, rs);
    __builtin_amdgcn_sched_barrier(0);
    uint8_t* lst = wbase + (size_t)wave * WAVE;
    float* ptab = reinterpret_cast<float*>(wbase + (size_t)wave * WAVE + LIST);
    if constexpr (RG) {
        // slots past a row find a valid table offset (channel 0) in every
        // entry no mask has written
        for (uint32_t i = (uint32_t)L; i < LIST / 16u; i += 64u) reinterpret_cast<uint4*>(lst)[i] = make_uint4(0, 0, 0, 0);
    } else if constexpr (TFIX == 0) {
        // the entries the score loop reads past a row that no mask writes:
        // the row's slack (from the 8-byte group holding entry T on; the
        // masks rewrite those below T) and the spare entries after the last
        // row; all start at a valid table offset (channel 0)
        for (uint32_t e = (uint32_t)T & ~3u; e < lstride; e += 4u)
            reinterpret_cast<uint2*>(lst)[((uint32_t)L * lstride + e) >> 2] = make_uint2(0, 0);
        if (L < 4) reinterpret_cast<uint2*>(lst)[16u * lstride + (uint32_t)L] = make_uint2(0, 0);
    }
    // the first tile's slot list needs only its masks: build it before
    // waiting for the table, then request the tile's V rows
    build_list(mw, lst, L, lstride);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (VB) {
        vbs.rvo = vblock_recovery(rvq[0], rvq[1]);
        vbs.kbits = load_v_tile_blocks(vbh, vbs.vm, a.nbv, tf0, ntf0, L >> 4, L & 15, vr);
    } else {
        load_v_tile(vbh, tf0, ntf0, L >> 4, L & 15, vr);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int j = tid + i * DECODE_FAST_THREADS;
        if (j < 128 * G) {
            const float qv = bf16_to_f32(qb[i]) * a.qscale;
            *reinterpret_cast<float*>(tab + qtab_offset<G>((uint32_t)(j & 127), (uint32_t)(j >> 7))) = qv;
            if (SMODE) qn[(j & 127) * G + (j >> 7)] = qv * ns;     // ns belongs to channel tid & 127 == j & 127
        }
    }
    if (tid < 128) *reinterpret_cast<float*>(tab + fast_rtab(G) + 16u * (uint32_t)tid) = rv;
    __syncthreads();

    // q' . r per head
    float cq[G];
    {
        const QV<G> e0 = load_qrow<G>(tab, 16u * (uint32_t)L);
        const QV<G> e1 = load_qrow<G>(tab, 16u * (uint32_t)(L + 64));
        const float r0 = *reinterpret_cast<const float*>(tab + fast_rtab(G) + 16u * (uint32_t)L);
        const float r1 = *reinterpret_cast<const float*>(tab + fast_rtab(G) + 16u * (uint32_t)(L + 64));
#pragma unroll
        for (int g = 0; g < G; ++g) cq[g] = wave_sum_dpp(e0.v[g] * r0 + e1.v[g] * r1);
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
        const int t1 = t0 + FAST_NW * DECODE_TILE, t2 = t1 + FAST_NW * DECODE_TILE;
        fast_tile<G, TB, TFIX, ODD, SMODE, false, true, RG, VB>(
            a, T, lstride, bh, tab, lst, ptab, vbh, cq, t0, min(DECODE_TILE, blk_end - t0),
            t1 < blk_end ? min(DECODE_TILE, blk_end - t1) : 0, L, mw, kr, vr, m_run, l_run, accm, qn, rs,
            t2 < blk_end ? min(DECODE_TILE, blk_end - t2) : 0, vbs);
    }
    for (int tile = wave + FAST_NW; tile < ntiles; tile += FAST_NW) {
        const int t0 = blk_begin + tile * DECODE_TILE;
        const int t1 = t0 + FAST_NW * DECODE_TILE, t2 = t1 + FAST_NW * DECODE_TILE;   // this wave's next two tiles
        uint4 vt[16];
        fast_tile<G, TB, TFIX, ODD, SMODE, true, false, RG, VB>(
            a, T, lstride, bh, tab, lst, ptab, vbh, cq, t0, min(DECODE_TILE, blk_end - t0),
            t1 < blk_end ? min(DECODE_TILE, blk_end - t1) : 0, L, mw, kr, vt, m_run, l_run, accm, qn, rs,
            t2 < blk_end ? min(DECODE_TILE, blk_end - t2) : 0, vbs);
    }

    float acc[G][8];
    combine_mf<G>(accm, acc);
    finish_block<G, DECODE_FAST_THREADS, true>(a, m_run, l_run, acc, wbase,
                                               reinterpret_cast<int*>(smem + TABLES), bh, b, h, split);
}

// Launch one variant, after checking that the block and split merge scratch
// (reused from the waves' regions after the tile loop) fits.
template <int G, int TB, int TFIX, bool ODD, int SMODE, bool RG, bool VB = false>
hipError_t launch_fast_variant(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
    using C = FastCfg<G, TB, TFIX, ODD, RG>;
    if (finish_scratch_bytes(G, DECODE_FAST_THREADS, a.nsplit) > (uint32_t)FAST_NW * C::WAVE)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_fast_kernel<G, TB, TFIX, ODD, SMODE, RG, VB>), grid, dim3(DECODE_FAST_THREADS), 0,
                       stream, a);
    return hipGetLastError();
}

// Runtime-T variants of one group size (VB: block-pruned V).
template <int G, bool VB>
hipError_t launch_fast_rt_v(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
    const bool odd = (a.T & 1) != 0;
    const int tb = decode_fast_bucket(a.T);
    switch (tb) {
        case 32: return odd ? launch_fast_variant<G, 32, 0, true, 0, false, VB>(a, grid, stream)
                            : launch_fast_variant<G, 32, 0, false, 0, false, VB>(a, grid, stream);
        case 64: return odd ? launch_fast_variant<G, 64, 0, true, 0, false, VB>(a, grid, stream)
                            : launch_fast_variant<G, 64, 0, false, 0, false, VB>(a, grid, stream);
        case 96: return odd ? launch_fast_variant<G, 96, 0, true, 0, false, VB>(a, grid, stream)
                            : launch_fast_variant<G, 96, 0, false, 0, false, VB>(a, grid, stream);
        case 128: return odd ? launch_fast_variant<G, 128, 0, true, 0, false, VB>(a, grid, stream)
                             : launch_fast_variant<G, 128, 0, false, 0, false, VB>(a, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

// Runtime-T and ragged variants of one group size.
template <int G>
hipError_t launch_fast_rt(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
    if (a.row_off) return launch_fast_variant<G, 128, 0, true, 0, true>(a, grid, stream);
    return launch_fast_rt_v<G, false>(a, grid, stream);
}

}  // namespace

}  // namespace spark
