// Observation-window token eviction (SnapKV style) on gfx950: the eviction
// stage that SparK's channel pruning is stacked on in the compacted-cache
// workload (SparK walkthrough section 4.1, where the method is combined with
// SnapKV; section 3.2 takes its observation window from the same idea).
//
// Per (b, KV head h), the R = G*W window query rows (head hG+g, position
// S-W+w, stacked in (g, w) order) score every cached token t <= S-W+w:
//     logit[r][t] = q_r . k_t / sqrt(D),   p[r][t] = softmax over t of logit[r]
//     score[t]    = sum over r of p[r][t]
// and the `keep` highest-scoring tokens (ties to the lower t) are kept in
// ascending t order, with their K and V rows gathered.
//
// The logits are a dense contraction (R x D times D x S), so they run on the
// matrix cores (v_mfma_f32_16x16x32_bf16) with q and k as exact bf16 and fp32
// accumulation. Two passes over K: (1) each row's max and sum of exp over its
// visible tokens (per chunk, then combined), (2) the normalised sum over rows.
// Then a radix select on the fp32 score bits and a gather.
#include "common.h"
#include "kernels.h"

namespace spark {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each wave owns EVICT_WAVE_ROWS window rows (two 16-row blocks); a block has
// one wave per 32 rows and all its waves walk the same tokens.
constexpr int MBW = EVICT_WAVE_ROWS / 16;

// The wave's window rows as MFMA A operands: q[mb][kb] holds rows
// r0 + 16 mb + (lane & 15), dims 32 kb + 8 (lane >> 4) .. +8 (rows past R
// are zero).
__device__ __forceinline__ void load_rows(const EvictArgs& a, int b, int h, int r0, int L, bf16x8 (&q)[MBW][4]) {
    const int G = a.N_q / a.N_kv;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        const int r = r0 + 16 * mb + (L & 15);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (r < a.R) {
                const int g = r / a.W, w = r % a.W;
                const uint16_t* src = a.q_win + (((size_t)b * a.N_q + (size_t)h * G + g) * a.W + w) * 128 + 32 * kb +
                                      8 * (L >> 4);
                v = *reinterpret_cast<const uint4*>(src);
            }
            q[mb][kb] = __builtin_bit_cast(bf16x8, v);
        }
    }
}

// K tiles of EVICT_TILE tokens pass through LDS: every wave of the block
// loads a quarter of the next tiles into registers (coalesced 16-byte chunks:
// lanes 0-15 read one 256-byte row), writes it to one of two LDS buffers,
// and after a barrier all waves read their MFMA B operands from it. Rows are
// padded to 272 bytes to spread the B-operand reads over the banks.
constexpr int TILE_ROW = 128 * 2 + 16;
constexpr int TILE_BYTES = EVICT_TILE * TILE_ROW;
constexpr int NWV = EVICT_MAX_ROWS / EVICT_WAVE_ROWS;
constexpr int CPL = EVICT_TILE * 16 / (NWV * 64);   // 16-byte chunks per lane per tile

// (nontemporal requests: each wave reads whole 256-byte K rows once per pass;
// streaming them past the L2 took the stage 365 -> 331 us at B=8, S=32K)
__device__ __forceinline__ void fetch_tile(const EvictArgs& a, const uint16_t* kbh, int t0, int tid, u32x4 (&r)[CPL]) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = tid + j * NWV * 64;             // chunk of the tile: token c >> 4, dims 8 (c & 15)
        const int t = min(t0 + (c >> 4), a.S - 1);
        r[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbh + (size_t)t * 128 + 8 * (c & 15)));
    }
}

__device__ __forceinline__ void stash_tile(unsigned char* buf, int tid, const u32x4 (&r)[CPL]) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = tid + j * NWV * 64;
        *reinterpret_cast<u32x4*>(buf + (c >> 4) * TILE_ROW + 16 * (c & 15)) = r[j];
    }
}

// Logits times log2(e)/sqrt(D) of the wave's rows against tokens t0 + 16 n ..
// +15 of the LDS tile: s[mb][e] is row r0 + 16 mb + 4 (lane >> 4) + e, token
// t0 + 16 n + (lane & 15); tokens past S or not visible to the row are -inf.
__device__ __forceinline__ void logits16(const EvictArgs& a, const bf16x8 (&q)[MBW][4], const unsigned char* buf, int n,
                                         int r0, int t0, int L, f32x4 (&s)[MBW]) {
    bf16x8 kv[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        kv[kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(buf + (16 * n + (L & 15)) * TILE_ROW + 64 * kb +
                                                                           16 * (L >> 4)));
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q[mb][kb], kv[kb], c, 0, 0, 0);
        s[mb] = c * a.scale_log2;
    }
    const int tn = t0 + 16 * n;
    // visibility: row r (window position w = r % W) sees t <= S - W + w
    if (tn + 15 > a.S - a.W) {
        const int t = tn + (L & 15);
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + 16 * mb + 4 * (L >> 4) + e;
                if (t >= a.S || r >= a.R || t > a.S - a.W + r % a.W) s[mb][e] = -INFINITY;
            }
    }
}

// Walk the block's chunk tile by tile: the next two tiles are in flight in
// registers while the current one is used from LDS. f.tile(buf, t0) handles
// the EVICT_TILE tokens from t0 of the tile in buf.
template <typename F>
__device__ __forceinline__ void walk_tiles(const EvictArgs& a, const uint16_t* kbh, int tb, int te, unsigned char* lds,
                                           F& f) {
    const int tid = threadIdx.x;
    u32x4 ra[CPL], rb[CPL];
    fetch_tile(a, kbh, tb, tid, ra);
    if (tb + EVICT_TILE < te) fetch_tile(a, kbh, tb + EVICT_TILE, tid, rb);
    unsigned char* b0 = lds;
    unsigned char* b1 = lds + TILE_BYTES;
    for (int t0 = tb; t0 < te; t0 += 2 * EVICT_TILE) {
        stash_tile(b0, tid, ra);
        if (t0 + 2 * EVICT_TILE < te) fetch_tile(a, kbh, t0 + 2 * EVICT_TILE, tid, ra);
        __syncthreads();
        f.tile(b0, t0);
        if (t0 + EVICT_TILE >= te) break;
        stash_tile(b1, tid, rb);
        if (t0 + 3 * EVICT_TILE < te) fetch_tile(a, kbh, t0 + 3 * EVICT_TILE, tid, rb);
        __syncthreads();
        f.tile(b1, t0 + EVICT_TILE);
    }
}

// (m, l) of two partial softmax sums over disjoint token sets, base 2.
__device__ __forceinline__ void ml_merge(float& m, float& l, float mo, float lo) {
    const float mn = fmaxf(m, mo);
    l = l * exp2f(m - mn) + lo * exp2f(mo - mn);
    m = mn;
}

}  // namespace

// Pass 1: per (b*N_kv + h, chunk of EVICT_CHUNK tokens), each row's max and
// sum of exp2 over the chunk's visible tokens.
__global__ void __launch_bounds__(NWV * 64) evict_stats_kernel(const EvictArgs a) {
    __shared__ __align__(16) unsigned char lds[2 * TILE_BYTES];
    const int bh = blockIdx.y, chunk = blockIdx.x;
    const int b = bh / a.N_kv, h = bh % a.N_kv;
    const int L = threadIdx.x & 63;
    const int r0 = (threadIdx.x >> 6) * EVICT_WAVE_ROWS;
    bf16x8 q[MBW][4];
    load_rows(a, b, h, r0, L, q);
    const uint16_t* kbh = a.k + (size_t)bh * a.S * 128;
    // running (m, l) per lane for its rows and its token column; a finite
    // start keeps fully masked columns free of inf - inf
    float m[MBW][4], l[MBW][4];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) { m[mb][e] = -1e30f; l[mb][e] = 0.f; }
    const int tb = chunk * EVICT_CHUNK, te = min(a.S, tb + EVICT_CHUNK);
    struct Stats {
        const EvictArgs& a;
        const bf16x8 (&q)[MBW][4];
        float (&m)[MBW][4];
        float (&l)[MBW][4];
        int r0, L, te;
        // the tile's logits first, then one rescale per row and tile
        __device__ __forceinline__ void tile(const unsigned char* buf, int t0) {
            constexpr int NB = EVICT_TILE / 16;
            f32x4 s[NB][MBW];
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                if (t0 + 16 * n < te) logits16(a, q, buf, n, r0, t0, L, s[n]);
                else {
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb) s[n][mb] = (f32x4){-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                }
            }
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float mn = m[mb][e];
#pragma unroll
                    for (int n = 0; n < NB; ++n) mn = fmaxf(mn, s[n][mb][e]);
                    // the hardware exp2 (v_exp_f32, about 1 ulp, no denormal
                    // rescaling): every term is at most 1 and the sum at least 1
                    float acc = l[mb][e] * __builtin_amdgcn_exp2f(m[mb][e] - mn);
#pragma unroll
                    for (int n = 0; n < NB; ++n) acc += __builtin_amdgcn_exp2f(s[n][mb][e] - mn);
                    l[mb][e] = acc;
                    m[mb][e] = mn;
                }
        }
    } f{a, q, m, l, r0, L, te};
    walk_tiles(a, kbh, tb, te, lds, f);
    // combine the 16 token columns (lanes with the same lane >> 4)
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const float mo = __shfl_xor(m[mb][e], o, 64);
                const float lo = __shfl_xor(l[mb][e], o, 64);
                ml_merge(m[mb][e], l[mb][e], mo, lo);
            }
        }
    if ((L & 15) == 0) {
        float* out = a.part + ((size_t)bh * gridDim.x + chunk) * EVICT_MAX_ROWS * 2;
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + 16 * mb + 4 * (L >> 4) + e;
                out[2 * r] = m[mb][e];
                out[2 * r + 1] = l[mb][e];
            }
    }
}

// Per (b*N_kv + h, row): combine the chunks' (m, l) in chunk order; store
// (M, 1 / L). Loads are issued eight chunks at a time.
__global__ void evict_combine_kernel(const EvictArgs a, int nchunk) {
    const int bh = blockIdx.x, r = threadIdx.x;
    if (r >= EVICT_MAX_ROWS) return;
    const float2* p = reinterpret_cast<const float2*>(a.part + (size_t)bh * nchunk * EVICT_MAX_ROWS * 2) + r;
    float m = -1e30f, l = 0.f;
    for (int c0 = 0; c0 < nchunk; c0 += 8) {
        float2 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = c0 + i < nchunk ? p[(size_t)(c0 + i) * EVICT_MAX_ROWS] : make_float2(-1e30f, 0.f);
#pragma unroll
        for (int i = 0; i < 8; ++i) ml_merge(m, l, v[i].x, v[i].y);
    }
    a.rowstat[((size_t)bh * EVICT_MAX_ROWS + r) * 2] = m;
    a.rowstat[((size_t)bh * EVICT_MAX_ROWS + r) * 2 + 1] = l > 0.f ? 1.0f / l : 0.f;
}

// Pass 2: score[t] = sum over rows of exp2(s - M) / L for the chunk's tokens;
// each wave sums its rows, the waves' sums meet in LDS.
__global__ void __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(4))) evict_score_kernel(const EvictArgs a) {
    __shared__ __align__(16) unsigned char lds[2 * TILE_BYTES];
    // per tile, each wave's row sums of its 64 tokens, in two buffers by tile
    // parity: a tile's sums are added over the waves (and stored) after the
    // barrier that precedes the next tile, so 2 KiB of LDS suffice and four
    // blocks fit on a CU
    __shared__ float part[2][NWV][EVICT_TILE];
    const int bh = blockIdx.y, chunk = blockIdx.x;
    const int b = bh / a.N_kv, h = bh % a.N_kv;
    const int L = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = wave * EVICT_WAVE_ROWS;
    bf16x8 q[MBW][4];
    load_rows(a, b, h, r0, L, q);
    float M[MBW][4], iL[MBW][4];
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = r0 + 16 * mb + 4 * (L >> 4) + e;
            M[mb][e] = a.rowstat[((size_t)bh * EVICT_MAX_ROWS + r) * 2];
            iL[mb][e] = r < a.R ? a.rowstat[((size_t)bh * EVICT_MAX_ROWS + r) * 2 + 1] : 0.f;
        }
    const uint16_t* kbh = a.k + (size_t)bh * a.S * 128;
    const int tb = chunk * EVICT_CHUNK, te = min(a.S, tb + EVICT_CHUNK);
    float* sc = a.scores + (size_t)bh * a.S;
    struct Score {
        const EvictArgs& a;
        const bf16x8 (&q)[MBW][4];
        const float (&M)[MBW][4];
        const float (&iL)[MBW][4];
        float (*part)[NWV][EVICT_TILE];
        float* sc;
        int r0, L, wave, tb, te;
        // the previous tile's scores: its sums are complete after the barrier
        // that precedes this tile
        __device__ __forceinline__ void flush(int tp0) {
            const int i = threadIdx.x;
            if (i < EVICT_TILE && tp0 + i < te) {
                const int k = ((tp0 - tb) / EVICT_TILE) & 1;
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < NWV; ++w) v += part[k][w][i];
                sc[tp0 + i] = v;
            }
        }
        __device__ __forceinline__ void tile(const unsigned char* buf, int t0) {
            if (t0 > tb) flush(t0 - EVICT_TILE);
            float* out = part[((t0 - tb) / EVICT_TILE) & 1][wave];
#pragma unroll
            for (int n = 0; n < EVICT_TILE / 16; ++n) {
                if (t0 + 16 * n >= te) break;
                f32x4 s[MBW];
                logits16(a, q, buf, n, r0, t0, L, s);
                float acc = 0.f;
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc = fmaf(__builtin_amdgcn_exp2f(s[mb][e] - M[mb][e]), iL[mb][e], acc);
                // rows 4 (lane >> 4) + e of every block: add the four lane quarters
                acc = xor32_sum(xor16_sum(acc));
                if (L < 16) out[16 * n + L] = acc;
            }
        }
    } f{a, q, M, iL, part, sc, r0, L, wave, tb, te};
    walk_tiles(a, kbh, tb, te, lds, f);
    __syncthreads();
    if (te > tb) f.flush(tb + (te - tb - 1) / EVICT_TILE * EVICT_TILE);
}

// Exclusive prefix sum of v over the block (thread order), and the block
// total: a shuffle scan inside each wave, then the wave totals. Every thread
// of the block must call it.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wtot, uint32_t& total) {
    constexpr int NWV = NT / 64;
    const int tid = threadIdx.x, L = tid & 63, wave = tid >> 6;
    uint32_t s = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(s, o, 64);
        if (L >= o) s += t;
    }
    if (L == 63) wtot[wave] = s;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        const uint32_t t = wtot[w];
        off += w < wave ? t : 0u;
        tot += t;
    }
    __syncthreads();          // wtot may be reused by the next call
    total = tot;
    return off + s - v;
}

// Per (b*N_kv + h): the `keep` largest scores (fp32 >= 0, compared as their
// uint32 bits), ties to the lower t, written to idx in ascending t. The
// keep-th largest value theta is found bit by bit from the top by counting
// the values >= each candidate (one compare per value, wave sums, one
// barrier per bit); the search stops as soon as exactly `keep` values are >=
// the candidate. Then an ordered compaction: every value > theta, and the
// first values == theta in t order until `keep` are taken. Each thread owns a
// contiguous run of at most PER tokens, held in registers.
template <int PER>
__global__ void __launch_bounds__(EVICT_SELECT_THREADS) evict_select_kernel(const EvictArgs a) {
    constexpr int NT = EVICT_SELECT_THREADS;
    constexpr int NWV = NT / 64;
    __shared__ uint32_t wsum[2][NWV];
    __shared__ uint32_t wtot[NWV];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, L = tid & 63, wave = tid >> 6;
    const uint32_t* u = reinterpret_cast<const uint32_t*>(a.scores) + (size_t)bh * a.S;
    const int S = a.S;
    const int t_begin = min(S, tid * PER), n = min(S, t_begin + PER) - t_begin;
    uint32_t x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] = i < n ? u[t_begin + i] : 0u;
    const uint32_t keep = (uint32_t)a.keep;
    // theta: the largest v with #{x >= v} >= keep (values past n are 0 and
    // are never counted: a candidate always has a set bit)
    uint32_t v = 0;
    bool exact = false;
    for (int bit = 31, par = 0; bit >= 0; --bit, par ^= 1) {
        const uint32_t c = v | (1u << bit);
        uint32_t cnt = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) cnt += x[i] >= c ? 1u : 0u;
        const float cw = wave_sum_dpp((float)cnt);                   // exact: counts < 2^24
        if (L == 0) wsum[par][wave] = (uint32_t)cw;
        __syncthreads();
        uint32_t total = 0;
#pragma unroll
        for (int w = 0; w < NWV; ++w) total += wsum[par][w];
        if (total >= keep) {
            v = c;
            if (total == keep) { exact = true; break; }
        }
    }
    // with an exact count every value >= v is kept; otherwise the values > v
    // and the first (keep - #{x > v}) values == v in t order
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        n_gt += (i < n && x[i] > v) ? 1u : 0u;
        n_eq += (i < n && x[i] == v) ? 1u : 0u;
    }
    uint32_t eq_before = 0, take_eq = 0;
    if (!exact) {      // uniform
        uint32_t gt_total, eq_total;
        (void)block_excl_scan<NT>(n_gt, wtot, gt_total);
        eq_before = block_excl_scan<NT>(n_eq, wtot, eq_total);
        take_eq = keep - gt_total;
    } else {
        take_eq = 0xffffffffu;     // every value == v is kept
    }
    uint32_t n_keep = n_gt;
    {
        uint32_t e = eq_before;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (i < n && x[i] == v) { n_keep += e < take_eq ? 1u : 0u; ++e; }
    }
    uint32_t kept_total;
    uint32_t pos = block_excl_scan<NT>(n_keep, wtot, kept_total);
    int32_t* idx = a.idx + (size_t)bh * a.keep;
    uint32_t e = eq_before;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (i < n) {
            bool k = x[i] > v;
            if (x[i] == v) { k = e < take_eq; ++e; }
            if (k && pos < keep) idx[pos++] = t_begin + i;
        }
    }
}

// Caches longer than the register-held select takes (64 tokens a thread):
// the same search and compaction, with the scores read again from global
// memory (4 bytes a token; they stay in L2) at every step. The counts read
// them thread-interleaved, one request per 64 consecutive tokens of a wave;
// the ordered compaction reads each thread's contiguous run twice, for its
// counts and then for its writes.
__global__ void __launch_bounds__(EVICT_SELECT_THREADS) evict_select_long_kernel(const EvictArgs a) {
    constexpr int NT = EVICT_SELECT_THREADS;
    constexpr int NWV = NT / 64;
    __shared__ uint32_t wsum[2][NWV];
    __shared__ uint32_t wtot[NWV];
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, L = tid & 63, wave = tid >> 6;
    const uint32_t* u = reinterpret_cast<const uint32_t*>(a.scores) + (size_t)bh * a.S;
    const int S = a.S;
    const uint32_t keep = (uint32_t)a.keep;
    uint32_t v = 0;
    bool exact = false;
    for (int bit = 31, par = 0; bit >= 0; --bit, par ^= 1) {
        const uint32_t c = v | (1u << bit);
        uint32_t cnt = 0;
        for (int t = tid; t < S; t += NT) cnt += u[t] >= c ? 1u : 0u;
        const float cw = wave_sum_dpp((float)cnt);                   // exact: counts < 2^24
        if (L == 0) wsum[par][wave] = (uint32_t)cw;
        __syncthreads();
        uint32_t total = 0;
#pragma unroll
        for (int w = 0; w < NWV; ++w) total += wsum[par][w];
        if (total >= keep) {
            v = c;
            if (total == keep) { exact = true; break; }
        }
    }
    const int per = (S + NT - 1) / NT;
    const int t_begin = min(S, tid * per), t_end = min(S, t_begin + per);
    uint32_t n_gt = 0, n_eq = 0;
    for (int t = t_begin; t < t_end; ++t) {
        const uint32_t x = u[t];
        n_gt += x > v ? 1u : 0u;
        n_eq += x == v ? 1u : 0u;
    }
    uint32_t eq_before = 0, take_eq = 0;
    if (!exact) {      // uniform
        uint32_t gt_total, eq_total;
        (void)block_excl_scan<NT>(n_gt, wtot, gt_total);
        eq_before = block_excl_scan<NT>(n_eq, wtot, eq_total);
        take_eq = keep - gt_total;
    } else {
        take_eq = 0xffffffffu;     // every value == v is kept
    }
    const uint32_t n_take = n_eq == 0 ? 0u
                          : eq_before >= take_eq ? 0u
                          : min(n_eq, take_eq - eq_before);
    uint32_t kept_total;
    uint32_t pos = block_excl_scan<NT>(n_gt + n_take, wtot, kept_total);
    int32_t* idx = a.idx + (size_t)bh * a.keep;
    uint32_t e = eq_before;
    for (int t = t_begin; t < t_end; ++t) {
        const uint32_t x = u[t];
        bool k = x > v;
        if (x == v) { k = e < take_eq; ++e; }
        if (k && pos < keep) idx[pos++] = t;
    }
}

// K and V rows of the kept tokens: one 16-byte chunk per thread.
__global__ void evict_gather_kernel(const EvictArgs a) {
    const size_t n = (size_t)a.BH * a.keep * 16;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        const size_t row = i >> 4;                  // bh * keep + j
        const int c = (int)(i & 15);
        const size_t bh = row / a.keep;
        const int t = min(max(a.idx[row], 0), a.S - 1);   // indices come from the select kernel
        const size_t src = ((size_t)bh * a.S + t) * 128 + 8 * c;
        reinterpret_cast<uint4*>(a.k_out)[row * 16 + c] = *reinterpret_cast<const uint4*>(a.k + src);
        reinterpret_cast<uint4*>(a.v_out)[row * 16 + c] = *reinterpret_cast<const uint4*>(a.v + src);
    }
}

hipError_t launch_evict(const EvictArgs& a, hipStream_t stream) {
    const int nchunk = (a.S + EVICT_CHUNK - 1) / EVICT_CHUNK;
    const dim3 blk(NWV * 64);
    hipLaunchKernelGGL(evict_stats_kernel, dim3(nchunk, a.BH), blk, 0, stream, a);
    hipLaunchKernelGGL(evict_combine_kernel, dim3(a.BH), dim3(EVICT_MAX_ROWS), 0, stream, a, nchunk);
    hipLaunchKernelGGL(evict_score_kernel, dim3(nchunk, a.BH), blk, 0, stream, a);
    const int per = (a.S + EVICT_SELECT_THREADS - 1) / EVICT_SELECT_THREADS;
    if (per <= 8) hipLaunchKernelGGL(evict_select_kernel<8>, dim3(a.BH), dim3(EVICT_SELECT_THREADS), 0, stream, a);
    else if (per <= 32) hipLaunchKernelGGL(evict_select_kernel<32>, dim3(a.BH), dim3(EVICT_SELECT_THREADS), 0, stream, a);
    else if (per <= 64) hipLaunchKernelGGL(evict_select_kernel<64>, dim3(a.BH), dim3(EVICT_SELECT_THREADS), 0, stream, a);
    else if (a.S <= EVICT_MAX_S_LONG)
        hipLaunchKernelGGL(evict_select_long_kernel, dim3(a.BH), dim3(EVICT_SELECT_THREADS), 0, stream, a);
    else return hipErrorInvalidValue;
    if (a.k_out != nullptr) {
        const size_t n = (size_t)a.BH * a.keep * 16;
        const int blocks = (int)((n + 255) / 256 < 65535 ? (n + 255) / 256 : 65535);
        hipLaunchKernelGGL(evict_gather_kernel, dim3(blocks), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

size_t evict_part_floats(int BH, int S) {
    const size_t nchunk = (size_t)(S + EVICT_CHUNK - 1) / EVICT_CHUNK;
    return (size_t)BH * nchunk * EVICT_MAX_ROWS * 2;
}

}  // namespace spark
