// Decode attention over the SparK pruned key cache on gfx950 (walkthrough
// section 3.3 and Fig. 3 decode half): every pruned channel of a cached key
// takes the recovery value r_j, then softmax(q K_hat^T * scale) V runs over the
// dense V.
//
// The score is evaluated in its sparse form
//     q . k_hat_t = q . r + sum over kept j of q^j (k_tj - r_j),
// so each token costs G*T multiply-adds instead of G*D, and the kept channel
// indices come straight from the mask bits.
//
// Work split (flash-decoding style): grid = (nsplit, B*N_kv). A block of 4
// waves owns `chunk` consecutive tokens of one (b, KV head) and all G query
// heads of its group, so every byte of packed K, mask and V is read once per
// step. Each wave walks 64-token tiles:
//   * scores with one lane per token; the packed rows of the tile are staged
//     in LDS with 16-byte loads and read back per lane;
//   * online softmax (base-2, scale folded into q) with wave-wide max;
//   * P.V with lane = (token mod 4, 8-channel slice of d): each lane issues
//     16-byte V loads, 4 tokens per load instruction per wave.
// Partials (m, l, acc) of the 4 waves are merged in LDS; the last block of a
// (b, KV head) to finish (device-scope counter) merges all splits and writes
// the fp32 output, then resets its counter to zero.
#include "common.h"
#include "kernels.h"

namespace spark {

namespace {

template <int G>
struct QRow { float v[G]; };

}  // namespace

uint32_t decode_stage_bytes(int T) {
    // 64 rows of T bf16 plus up to 7 elements of 16-byte misalignment, whole 16-byte chunks
    const uint32_t elems = (uint32_t)DECODE_TILE * (uint32_t)T + 8u;
    return ((elems * 2u) + 15u) & ~15u;
}

size_t decode_lds_bytes(int G, int T) {
    const size_t tables = (size_t)128 * G * 4 + 128 * 4;
    const size_t per_wave = (size_t)DECODE_TILE * G * 4 + decode_stage_bytes(T);
    const size_t waves = DECODE_THREADS / 64;
    const size_t combine = waves * ((size_t)2 * G + (size_t)G * 128) * 4;
    const size_t dyn = waves * per_wave > combine + waves * (size_t)DECODE_TILE * G * 4
                           ? waves * per_wave : combine + waves * (size_t)DECODE_TILE * G * 4;
    return tables + dyn;
}

template <int G>
__global__ void __launch_bounds__(DECODE_THREADS)
decode_kernel(const DecodeArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = DECODE_THREADS / 64;
    float* qtab = reinterpret_cast<float*>(smem);              // [128][G], scaled by qscale
    float* rtab = qtab + 128 * G;                              // [128]
    float* ptab_all = rtab + 128;                              // [NW][64][G]
    unsigned char* stage_all = reinterpret_cast<unsigned char*>(ptab_all + NW * DECODE_TILE * G);

    const int bh = blockIdx.y;
    const int split = blockIdx.x;
    const int N_kv = a.N_kv;
    const int b = bh / N_kv, h = bh % N_kv;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int L = tid & 63;
    const int S = a.S, T = a.T;

    // ---- tables: q of the G heads (scaled) and r
    for (int i = tid; i < 128 * G; i += DECODE_THREADS) {
        const int g = i >> 7, j = i & 127;
        const uint16_t qb = a.q[((size_t)b * a.N_q + (size_t)h * G + g) * 128 + j];
        qtab[j * G + g] = bf16_to_f32(qb) * a.qscale;
    }
    if (tid < 128) rtab[tid] = a.r[(size_t)bh * 128 + tid];
    __syncthreads();

    // c_g = q'_g . r (the score of an all-pruned key)
    float cq[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        cq[g] = wave_sum(qtab[L * G + g] * rtab[L] + qtab[(L + 64) * G + g] * rtab[L + 64]);

    float* ptab = ptab_all + wave * DECODE_TILE * G;
    unsigned char* stage = stage_all + (size_t)wave * a.lds_stage_bytes;
    const uint16_t* stage16 = reinterpret_cast<const uint16_t*>(stage);

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

    const uint16_t* vbh = a.v + (size_t)bh * S * 128;
    const uint32_t* mbh = a.mask + (size_t)bh * S * 4;

    for (int tile = wave; tile < ntiles; tile += NW) {
        const int t0 = blk_begin + tile * DECODE_TILE;
        const int nt = min(DECODE_TILE, blk_end - t0);

        // -- loads: packed rows (to LDS), masks, V
        const size_t e0 = ((size_t)bh * S + t0) * (size_t)T;
        const size_t ea = e0 & ~(size_t)7;
        const int shift = (int)(e0 - ea);
        const size_t e1 = e0 + (size_t)nt * T;
        const int nchunks = (int)((e1 - ea + 7) >> 3);
        uint4 pk[4];
        int npk = 0;
        if (T > 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = L + 64 * u;
                pk[u] = make_uint4(0, 0, 0, 0);
                if (c < nchunks) {
                    const size_t ce = ea + (size_t)c * 8;
                    if (ce + 8 <= a.packed_elems) {
                        pk[u] = *reinterpret_cast<const uint4*>(a.packed + ce);
                    } else {
                        uint16_t tmp[8];
#pragma unroll
                        for (int x = 0; x < 8; ++x) tmp[x] = (ce + x < a.packed_elems) ? a.packed[ce + x] : 0;
                        pk[u] = make_uint4(tmp[0] | ((uint32_t)tmp[1] << 16), tmp[2] | ((uint32_t)tmp[3] << 16),
                                           tmp[4] | ((uint32_t)tmp[5] << 16), tmp[6] | ((uint32_t)tmp[7] << 16));
                    }
                }
            }
            npk = 4;
        }
        uint4 mw = make_uint4(0, 0, 0, 0);
        if (L < nt) mw = *reinterpret_cast<const uint4*>(mbh + (size_t)(t0 + L) * 4);
        uint4 vr[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tok = 4 * i + tau;
            vr[i] = make_uint4(0, 0, 0, 0);
            if (tok < nt) vr[i] = *reinterpret_cast<const uint4*>(vbh + (size_t)(t0 + tok) * 128 + oct * 8);
        }

        // -- packed rows into LDS (chunks beyond the first 256 loaded in a loop)
        if (npk) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = L + 64 * u;
                if (c < nchunks) reinterpret_cast<uint4*>(stage)[c] = pk[u];
            }
            for (int c = L + 256; c < nchunks; c += 64) {
                const size_t ce = ea + (size_t)c * 8;
                uint4 x;
                if (ce + 8 <= a.packed_elems) {
                    x = *reinterpret_cast<const uint4*>(a.packed + ce);
                } else {
                    uint16_t tmp[8];
                    for (int y = 0; y < 8; ++y) tmp[y] = (ce + y < a.packed_elems) ? a.packed[ce + y] : 0;
                    x = make_uint4(tmp[0] | ((uint32_t)tmp[1] << 16), tmp[2] | ((uint32_t)tmp[3] << 16),
                                   tmp[4] | ((uint32_t)tmp[5] << 16), tmp[6] | ((uint32_t)tmp[7] << 16));
                }
                reinterpret_cast<uint4*>(stage)[c] = x;
            }
        }
        wave_lds_sync();

        // -- scores, one lane per token
        float s[G];
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = 0.f;
        if (L < nt) {
            const uint16_t* row = stage16 + shift + L * T;
            int rho = 0;
            const uint32_t words[4] = {mw.x, mw.y, mw.z, mw.w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t m = words[w];
                while (m) {
                    const int j = 32 * w + __builtin_ctz(m);
                    m &= m - 1;
                    const float e = bf16_to_f32(row[rho++]) - rtab[j];
                    const QRow<G> qv = *reinterpret_cast<const QRow<G>*>(qtab + j * G);
#pragma unroll
                    for (int g = 0; g < G; ++g) s[g] = fmaf(qv.v[g], e, s[g]);
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) s[g] += cq[g];
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) s[g] = -INFINITY;
        }

        // -- online softmax (base 2)
        float alpha[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mt = wave_max(s[g]);
            const float mn = fmaxf(m_run[g], mt);
            alpha[g] = exp2f(m_run[g] - mn);
            const float p = exp2f(s[g] - mn);
            l_run[g] = l_run[g] * alpha[g] + p;
            m_run[g] = mn;
            ptab[L * G + g] = p;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] *= alpha[g];
        wave_lds_sync();

        // -- P.V
#pragma unroll
        for (int i = 0; i < 16; ++i) {
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
        wave_lds_sync();
    }

    // ---- wave partial: reduce acc over the 4 token phases, l over lanes
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = acc[g][e];
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            acc[g][e] = x;
        }
        l_run[g] = wave_sum(l_run[g]);
    }
    __syncthreads();   // staging no longer needed: reuse it for the block merge
    float* wm = reinterpret_cast<float*>(stage_all);           // [NW][G]
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

    float* pml = a.part_ml + ((size_t)bh * a.nsplit + split) * 2 * G;
    float* pacc = a.part_acc + ((size_t)bh * a.nsplit + split) * G * 128;
    for (int i = tid; i < G * 128; i += DECODE_THREADS) {
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
        pacc[i] = x;
        if (d == 0) { pml[g] = M; pml[G + g] = l; }
    }

    // ---- last block of this (b, KV head) merges all splits
    __shared__ int s_last;
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(a.counters + bh, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(a.nsplit - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float* ml_bh = a.part_ml + (size_t)bh * a.nsplit * 2 * G;
    const float* acc_bh = a.part_acc + (size_t)bh * a.nsplit * G * 128;
    for (int i = tid; i < G * 128; i += DECODE_THREADS) {
        const int g = i >> 7, d = i & 127;
        float M = -INFINITY;
        for (int sp = 0; sp < a.nsplit; ++sp) M = fmaxf(M, ml_bh[sp * 2 * G + g]);
        float x = 0.f, l = 0.f;
        for (int sp = 0; sp < a.nsplit; ++sp) {
            const float ms = ml_bh[sp * 2 * G + g];
            const float f = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
            x += acc_bh[(size_t)sp * G * 128 + i] * f;
            l += ml_bh[sp * 2 * G + G + g] * f;
        }
        a.out[((size_t)b * a.N_q + (size_t)h * G + g) * 128 + d] = x / l;
    }
    if (tid == 0) __hip_atomic_store(a.counters + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_decode(const DecodeArgs& a, int G, int BH, hipStream_t stream) {
    const dim3 grid(a.nsplit, BH), block(DECODE_THREADS);
    const size_t lds = decode_lds_bytes(G, a.T);
    const void* fn = nullptr;
    switch (G) {
        case 1: fn = reinterpret_cast<const void*>(&decode_kernel<1>); break;
        case 2: fn = reinterpret_cast<const void*>(&decode_kernel<2>); break;
        case 4: fn = reinterpret_cast<const void*>(&decode_kernel<4>); break;
        case 8: fn = reinterpret_cast<const void*>(&decode_kernel<8>); break;
        default: return hipErrorInvalidValue;
    }
    if (lds > 65536) {
        // LDS above 64 KiB per workgroup must be requested explicitly (160 KiB per CU on gfx950)
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    switch (G) {
        case 1: hipLaunchKernelGGL(decode_kernel<1>, grid, block, lds, stream, a); break;
        case 2: hipLaunchKernelGGL(decode_kernel<2>, grid, block, lds, stream, a); break;
        case 4: hipLaunchKernelGGL(decode_kernel<4>, grid, block, lds, stream, a); break;
        default: hipLaunchKernelGGL(decode_kernel<8>, grid, block, lds, stream, a); break;
    }
    return hipGetLastError();
}

__global__ void fill_u32_kernel(uint32_t* p, uint32_t value, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = value;
}

}  // namespace spark
