// C ABI of libspark.so (declared in include/spark.h): host-side argument
// checks, workspace layout and kernel launches.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/spark.h"
#include "kernels.h"

using namespace spark;

namespace {

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int kept_or_neg(int D, float lambda) {
    if (D < 1 || !(lambda >= 0.0f && lambda <= 1.0f)) return -1;
    return (int)floor((1.0 - (double)lambda) * (double)D + 0.5);
}

int check_group(int N_q, int N_kv) {
    if (N_q < 1 || N_kv < 1 || N_q % N_kv != 0) return SPARK_EINVAL;
    const int G = N_q / N_kv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return SPARK_EUNSUPPORTED;
    return SPARK_OK;
}

// prefill workspace: part_sum double [BH][nblk][128] | part_cnt int32 [BH][nblk][128] |
// part_pruned double [BH][nblk][2] (sum of the pruned saliency, sum of its squares) |
// gid uint8 [BH][128] (SparK-g channel groups) | blk int32 [BH][nblk] (SparK-p block totals, then bases)
struct PrefillWs {
    double* sum;
    int32_t* cnt;
    double* pruned;
    uint8_t* gid;
    int32_t* blk;
    size_t bytes;
    int nblk;
};

PrefillWs prefill_layout(void* ws, int B, int S, int N_kv) {
    PrefillWs w{};
    const size_t BH = (size_t)B * N_kv;
    w.nblk = (S + PRUNE_TOKENS_PER_BLOCK - 1) / PRUNE_TOKENS_PER_BLOCK;
    const size_t n = BH * (size_t)w.nblk;
    const size_t s_sum = round_up(n * 128 * sizeof(double), 256);
    const size_t s_cnt = round_up(n * 128 * sizeof(int32_t), 256);
    const size_t s_pr = round_up(n * 2 * sizeof(double), 256);
    char* base = static_cast<char*>(ws);
    w.sum = reinterpret_cast<double*>(base);
    w.cnt = reinterpret_cast<int32_t*>(base + s_sum);
    w.pruned = reinterpret_cast<double*>(base + s_sum + s_cnt);
    w.gid = reinterpret_cast<uint8_t*>(base + s_sum + s_cnt + s_pr);
    const size_t s_gid = round_up(BH * 128, 256);
    w.blk = reinterpret_cast<int32_t*>(base + s_sum + s_cnt + s_pr + s_gid);
    w.bytes = s_sum + s_cnt + s_pr + s_gid + round_up(n * sizeof(int32_t), 256);
    return w;
}

// About `blocks` blocks in all (256: one 8-wave block per CU for the fast
// kernel; 512: two 4-wave blocks per CU for the generic one), but never fewer
// tiles per block than the block has waves: with few (b, KV head) pairs (a
// tensor-parallel shard of one KV head, say) more splits would leave waves
// without work.
int auto_splits(int BH, int S, int blocks, int waves) {
    const int max_splits = (S + DECODE_TILE * waves - 1) / (DECODE_TILE * waves);
    int want = (blocks + BH - 1) / BH;
    if (want < 1) want = 1;
    if (want > max_splits) want = max_splits;
    return want;
}

// decode: the number of splits actually launched and the tokens per split
void decode_plan(int BH, int S, int splits, int* nsplit, int* chunk, int blocks = 256,
                 int waves = DECODE_FAST_THREADS / 64) {
    int n = splits > 0 ? splits : auto_splits(BH, S, blocks, waves);
    const int max_splits = (S + DECODE_TILE - 1) / DECODE_TILE;
    if (n > max_splits) n = max_splits;
    if (n > DECODE_MAX_SPLITS) n = DECODE_MAX_SPLITS;
    int c = (S + n - 1) / n;
    c = (c + DECODE_TILE - 1) / DECODE_TILE * DECODE_TILE;
    *chunk = c;
    *nsplit = (S + c - 1) / c;
}

size_t decode_ws_bytes(int BH, int G, int nsplit) {
    return SPARK_DECODE_COUNTER_BYTES + round_up((size_t)BH * nsplit * 2 * G * sizeof(float), 256) +
           round_up((size_t)BH * nsplit * G * 128 * sizeof(float), 256);
}

int hip_status(hipError_t e) { return e == hipSuccess ? SPARK_OK : SPARK_EHIP; }

}  // namespace

extern "C" {

int spark_num_kept(int D, float lambda) { return kept_or_neg(D, lambda); }

int spark_num_kept_grouped(int D, int ngroups, const float* ratios) {
    if (D < 1 || ngroups < 1 || ngroups > SPARK_MAX_GROUPS || D % ngroups || !ratios) return -1;
    int T = 0;
    for (int i = 0; i < ngroups; ++i) {
        const int t = kept_or_neg(D / ngroups, ratios[i]);
        if (t < 0) return -1;
        T += t;
    }
    return T;
}

int spark_num_kept_vblocks(int D, float lambda_v) {
    if (D < SPARK_VBLOCK || D % SPARK_VBLOCK) return -1;
    return kept_or_neg(D / SPARK_VBLOCK, lambda_v);
}

size_t spark_vblock_mask_stride(int S) { return S < 1 ? 0 : vblock_mask_stride(S); }

const char* spark_strerror(int status) {
    switch (status) {
        case SPARK_OK: return "ok";
        case SPARK_EINVAL: return "invalid argument";
        case SPARK_EUNSUPPORTED: return "unsupported size (D must be 128; N_q/N_kv in {1,2,4,8})";
        case SPARK_EALIGN: return "misaligned pointer (tensors 16 B, workspace 256 B)";
        case SPARK_ENOSPACE: return "workspace too small";
        case SPARK_EHIP: return "HIP runtime error";
        case SPARK_ESCRATCH: return "problem needs more than the fixed scratch of spark_decode_attn_noalloc";
        default: return "unknown status";
    }
}

size_t spark_prefill_workspace_bytes(int B, int S, int N_kv, int D) {
    if (B < 1 || S < 1 || N_kv < 1 || D < 1) return 0;
    return prefill_layout(nullptr, B, S, N_kv).bytes;
}

size_t spark_decode_workspace_bytes(int B, int S, int N_q, int N_kv, int D, int splits) {
    if (B < 1 || S < 1 || N_kv < 1 || N_q < 1 || D < 1 || splits < 0 || N_q % N_kv) return 0;
    int nsplit, chunk;
    // sized for the larger of the two entry points' split plans
    decode_plan(B * N_kv, S, splits, &nsplit, &chunk, DECODE_GENERIC_BLOCKS, DECODE_THREADS / 64);
    return decode_ws_bytes(B * N_kv, N_q / N_kv, nsplit);
}

int spark_prefill_prune_cap(const void* q_win, const void* k, int B, int S, int S_cap, int N_q, int N_kv, int D,
                            float lambda, int window, int qagg, int recovery, float f_const,
                            void* k_packed, uint32_t* mask, float* chan_energy, float* r, int32_t* cnt,
                            void* ws, size_t ws_bytes, void* stream) {
    if (B < 1 || S < 1 || D < 1 || window < 1 || S_cap < S) return SPARK_EINVAL;
    const int T = kept_or_neg(D, lambda);
    if (T < 0) return SPARK_EINVAL;
    if (qagg != SPARK_QAGG_L2 && qagg != SPARK_QAGG_MEAN) return SPARK_EINVAL;
    if (recovery < SPARK_F_MEAN_RETAINED || recovery > SPARK_F_EXPONENTIAL) return SPARK_EINVAL;
    if (int e = check_group(N_q, N_kv)) return e;
    if (D != 128) return SPARK_EUNSUPPORTED;
    if (!q_win || !k || !mask || !chan_energy || !r || !ws || (T > 0 && !k_packed)) return SPARK_EINVAL;
    if (!aligned(q_win, 16) || !aligned(k, 16) || !aligned(mask, 16) || !aligned(chan_energy, 16) ||
        !aligned(r, 16) || (k_packed && !aligned(k_packed, 16)) || (cnt && !aligned(cnt, 16)) || !aligned(ws, 256))
        return SPARK_EALIGN;
    const PrefillWs w = prefill_layout(ws, B, S, N_kv);
    if (ws_bytes < w.bytes) return SPARK_ENOSPACE;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int BH = B * N_kv;
    hipLaunchKernelGGL(chan_energy_kernel, dim3(BH), dim3(256), 0, st,
                       static_cast<const uint16_t*>(q_win), chan_energy, N_q, N_kv, window, qagg);
    hipLaunchKernelGGL(select_pack_kernel<0>, dim3(w.nblk, BH), dim3(256), 0, st,
                       static_cast<const uint16_t*>(k), chan_energy, static_cast<uint16_t*>(k_packed), mask,
                       w.sum, w.cnt, w.pruned, S, T, w.nblk, recovery, static_cast<const uint8_t*>(nullptr),
                       GroupSpec{}, 0.0f, static_cast<int32_t*>(nullptr), static_cast<int32_t*>(nullptr), S_cap);
    hipLaunchKernelGGL(stats_reduce_kernel, dim3(BH, STATS_CH_BLOCKS), dim3(STATS_THREADS), 0, st,
                       w.sum, w.cnt, w.pruned, chan_energy, r, cnt, S, T, w.nblk, recovery, f_const, 0);
    return hip_status(hipGetLastError());
}

int spark_prefill_prune(const void* q_win, const void* k, int B, int S, int N_q, int N_kv, int D,
                        float lambda, int window, int qagg, int recovery, float f_const,
                        void* k_packed, uint32_t* mask, float* chan_energy, float* r, int32_t* cnt,
                        void* ws, size_t ws_bytes, void* stream) {
    return spark_prefill_prune_cap(q_win, k, B, S, S, N_q, N_kv, D, lambda, window, qagg, recovery, f_const,
                                   k_packed, mask, chan_energy, r, cnt, ws, ws_bytes, stream);
}

int spark_append_token(const void* k_new, const void* v_new, const float* chan_energy, int B, int N_kv, int D,
                       float lambda, int pos, int S_cap, void* k_packed, uint32_t* mask, void* v, void* stream) {
    if (B < 1 || N_kv < 1 || D < 1 || pos < 0 || pos >= S_cap) return SPARK_EINVAL;
    const int T = kept_or_neg(D, lambda);
    if (T < 0) return SPARK_EINVAL;
    if (D != 128) return SPARK_EUNSUPPORTED;
    if (!k_new || !v_new || !chan_energy || !mask || !v || (T > 0 && !k_packed)) return SPARK_EINVAL;
    if (!aligned(k_new, 4) || !aligned(v_new, 4) || !aligned(chan_energy, 4) || !aligned(mask, 16) ||
        !aligned(v, 16) || (k_packed && !aligned(k_packed, 16)))
        return SPARK_EALIGN;
    hipLaunchKernelGGL(append_token_kernel, dim3(B * N_kv), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), chan_energy,
                       static_cast<uint16_t*>(k_packed), mask, static_cast<uint16_t*>(v), T, pos, S_cap);
    return hip_status(hipGetLastError());
}

int spark_prefill_prune_v(const void* v, int B, int S, int N_kv, int D, float lambda_v, void* v_packed,
                          uint32_t* v_mask, float* r_v, int32_t* cnt, void* ws, size_t ws_bytes, void* stream) {
    if (B < 1 || S < 1 || N_kv < 1 || D < 1) return SPARK_EINVAL;
    const int T = kept_or_neg(D, lambda_v);
    if (T < 0) return SPARK_EINVAL;
    if (D != 128) return SPARK_EUNSUPPORTED;
    if (!v || !v_mask || !r_v || !ws || (T > 0 && !v_packed)) return SPARK_EINVAL;
    if (!aligned(v, 16) || !aligned(v_mask, 16) || !aligned(r_v, 16) || (v_packed && !aligned(v_packed, 16)) ||
        (cnt && !aligned(cnt, 16)) || !aligned(ws, 256))
        return SPARK_EALIGN;
    const PrefillWs w = prefill_layout(ws, B, S, N_kv);
    if (ws_bytes < w.bytes) return SPARK_ENOSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int BH = B * N_kv;
    hipLaunchKernelGGL(select_pack_kernel<0>, dim3(w.nblk, BH), dim3(256), 0, st,
                       static_cast<const uint16_t*>(v), static_cast<const float*>(nullptr),
                       static_cast<uint16_t*>(v_packed), v_mask, w.sum, w.cnt, w.pruned, S, T, w.nblk,
                       (int)SPARK_F_MEAN_RETAINED, static_cast<const uint8_t*>(nullptr), GroupSpec{}, 0.0f,
                       static_cast<int32_t*>(nullptr), static_cast<int32_t*>(nullptr), S);
    hipLaunchKernelGGL(stats_reduce_kernel, dim3(BH, STATS_CH_BLOCKS), dim3(STATS_THREADS), 0, st, w.sum, w.cnt, w.pruned,
                       static_cast<const float*>(nullptr), r_v, cnt, S, T, w.nblk, (int)SPARK_F_MEAN_RETAINED, 0.0f, 1);
    return hip_status(hipGetLastError());
}

int spark_prefill_prune_vblocks(const void* v, int B, int S, int N_kv, int D, float lambda_v, void* v_packed,
                                uint16_t* v_bmask, float* r_v, int32_t* cnt, void* ws, size_t ws_bytes, void* stream) {
    if (B < 1 || S < 1 || N_kv < 1 || D < 1) return SPARK_EINVAL;
    const int nb = spark_num_kept_vblocks(D, lambda_v);
    if (nb < 0) return SPARK_EINVAL;
    if (D != 128) return SPARK_EUNSUPPORTED;
    if ((size_t)B * N_kv > 65535) return SPARK_EUNSUPPORTED;
    if (!v || !v_bmask || !r_v || !ws || (nb > 0 && !v_packed)) return SPARK_EINVAL;
    if (!aligned(v, 16) || !aligned(v_bmask, 16) || !aligned(r_v, 16) || (v_packed && !aligned(v_packed, 16)) ||
        (cnt && !aligned(cnt, 16)) || !aligned(ws, 256))
        return SPARK_EALIGN;
    const PrefillWs w = prefill_layout(ws, B, S, N_kv);
    if (ws_bytes < w.bytes) return SPARK_ENOSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int BH = B * N_kv;
    hipLaunchKernelGGL(vblock_select_kernel, dim3(w.nblk, BH), dim3(256), 0, st, static_cast<const uint16_t*>(v),
                       static_cast<uint16_t*>(v_packed), v_bmask, w.sum, w.cnt, S, nb, w.nblk, S);
    hipLaunchKernelGGL(stats_reduce_kernel, dim3(BH, STATS_CH_BLOCKS), dim3(STATS_THREADS), 0, st, w.sum, w.cnt, w.pruned,
                       static_cast<const float*>(nullptr), r_v, cnt, S, SPARK_VBLOCK * nb, w.nblk,
                       (int)SPARK_F_MEAN_RETAINED, 0.0f, 1);
    return hip_status(hipGetLastError());
}

int spark_prefill_prune_grouped(const void* q_win, const void* k, int B, int S, int N_q, int N_kv, int D,
                                int ngroups, const float* ratios, int window, int qagg, int recovery, float f_const,
                                void* k_packed, uint32_t* mask, float* chan_energy, float* r, int32_t* cnt,
                                void* ws, size_t ws_bytes, void* stream) {
    if (B < 1 || S < 1 || D < 1 || window < 1) return SPARK_EINVAL;
    const int T = spark_num_kept_grouped(D, ngroups, ratios);
    if (T < 0) return SPARK_EINVAL;
    if (qagg != SPARK_QAGG_L2 && qagg != SPARK_QAGG_MEAN) return SPARK_EINVAL;
    if (recovery < SPARK_F_MEAN_RETAINED || recovery > SPARK_F_EXPONENTIAL) return SPARK_EINVAL;
    if (int e = check_group(N_q, N_kv)) return e;
    if (D != 128) return SPARK_EUNSUPPORTED;
    if (!q_win || !k || !mask || !chan_energy || !r || !ws || (T > 0 && !k_packed)) return SPARK_EINVAL;
    if (!aligned(q_win, 16) || !aligned(k, 16) || !aligned(mask, 16) || !aligned(chan_energy, 16) ||
        !aligned(r, 16) || (k_packed && !aligned(k_packed, 16)) || (cnt && !aligned(cnt, 16)) || !aligned(ws, 256))
        return SPARK_EALIGN;
    const PrefillWs w = prefill_layout(ws, B, S, N_kv);
    if (ws_bytes < w.bytes) return SPARK_ENOSPACE;
    GroupSpec grp{};
    grp.n = ngroups;
    grp.size = D / ngroups;
    for (int i = 0; i < ngroups; ++i) grp.T[i] = kept_or_neg(D / ngroups, ratios[i]);

    hipStream_t st = static_cast<hipStream_t>(stream);
    const int BH = B * N_kv;
    hipLaunchKernelGGL(chan_energy_kernel, dim3(BH), dim3(256), 0, st,
                       static_cast<const uint16_t*>(q_win), chan_energy, N_q, N_kv, window, qagg);
    hipLaunchKernelGGL(channel_groups_kernel, dim3(BH), dim3(128), 0, st, static_cast<const float*>(chan_energy),
                       w.gid, ngroups);
    hipLaunchKernelGGL(select_pack_kernel<1>, dim3(w.nblk, BH), dim3(256), 0, st,
                       static_cast<const uint16_t*>(k), static_cast<const float*>(chan_energy),
                       static_cast<uint16_t*>(k_packed), mask, w.sum, w.cnt, w.pruned, S, T, w.nblk, recovery,
                       static_cast<const uint8_t*>(w.gid), grp, 0.0f, static_cast<int32_t*>(nullptr),
                       static_cast<int32_t*>(nullptr), S);
    hipLaunchKernelGGL(stats_reduce_kernel, dim3(BH, STATS_CH_BLOCKS), dim3(STATS_THREADS), 0, st,
                       w.sum, w.cnt, w.pruned, chan_energy, r, cnt, S, T, w.nblk, recovery, f_const, 0);
    return hip_status(hipGetLastError());
}

int spark_prefill_prune_topp(const void* q_win, const void* k, int B, int S, int N_q, int N_kv, int D, float p,
                             int window, int qagg, int recovery, float f_const, void* k_packed, int32_t* row_off,
                             uint32_t* mask, float* chan_energy, float* r, int32_t* cnt, void* ws, size_t ws_bytes,
                             void* stream) {
    if (B < 1 || S < 1 || D < 1 || window < 1) return SPARK_EINVAL;
    if (!(p > 0.0f && p <= 1.0f)) return SPARK_EINVAL;
    if (qagg != SPARK_QAGG_L2 && qagg != SPARK_QAGG_MEAN) return SPARK_EINVAL;
    if (recovery < SPARK_F_MEAN_RETAINED || recovery > SPARK_F_EXPONENTIAL) return SPARK_EINVAL;
    if (int e = check_group(N_q, N_kv)) return e;
    if (D != 128) return SPARK_EUNSUPPORTED;
    if ((size_t)S * 128 > (size_t)INT32_MAX) return SPARK_EUNSUPPORTED;
    if (!q_win || !k || !k_packed || !row_off || !mask || !chan_energy || !r || !ws) return SPARK_EINVAL;
    if (!aligned(q_win, 16) || !aligned(k, 16) || !aligned(mask, 16) || !aligned(chan_energy, 16) ||
        !aligned(r, 16) || !aligned(k_packed, 16) || !aligned(row_off, 4) || (cnt && !aligned(cnt, 16)) ||
        !aligned(ws, 256))
        return SPARK_EALIGN;
    const PrefillWs w = prefill_layout(ws, B, S, N_kv);
    if (ws_bytes < w.bytes) return SPARK_ENOSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int BH = B * N_kv;
    // per-token counts go to row_off[t + 1] (as offsets of a (S + 1)-long row per head)
    hipLaunchKernelGGL(chan_energy_kernel, dim3(BH), dim3(256), 0, st,
                       static_cast<const uint16_t*>(q_win), chan_energy, N_q, N_kv, window, qagg);
    hipLaunchKernelGGL(select_pack_kernel<2>, dim3(w.nblk, BH), dim3(256), 0, st, static_cast<const uint16_t*>(k),
                       static_cast<const float*>(chan_energy), static_cast<uint16_t*>(nullptr), mask, w.sum, w.cnt,
                       w.pruned, S, -1, w.nblk, recovery, static_cast<const uint8_t*>(nullptr), GroupSpec{}, p,
                       row_off + 1, w.blk, S);
    hipLaunchKernelGGL(topp_scan_kernel, dim3(BH), dim3(64), 0, st, w.blk, w.nblk);
    hipLaunchKernelGGL(topp_pack_kernel, dim3(w.nblk, BH), dim3(256), 0, st, static_cast<const uint16_t*>(k),
                       static_cast<const uint32_t*>(mask), static_cast<uint16_t*>(k_packed), row_off,
                       static_cast<const int32_t*>(w.blk), S, w.nblk);
    hipLaunchKernelGGL(stats_reduce_kernel, dim3(BH, STATS_CH_BLOCKS), dim3(STATS_THREADS), 0, st,
                       w.sum, w.cnt, w.pruned, chan_energy, r, cnt, S, -1, w.nblk, recovery, f_const, 0);
    return hip_status(hipGetLastError());
}

int spark_stats(const void* k_packed, const uint32_t* mask, const float* chan_energy, const void* k_dense,
                int B, int S, int N_kv, int D, float lambda, int recovery, float f_const,
                float* r, int32_t* cnt, void* ws, size_t ws_bytes, void* stream) {
    if (B < 1 || S < 1 || N_kv < 1 || D < 1) return SPARK_EINVAL;
    const int T = kept_or_neg(D, lambda);
    if (T < 0) return SPARK_EINVAL;
    if (recovery < SPARK_F_MEAN_RETAINED || recovery > SPARK_F_EXPONENTIAL) return SPARK_EINVAL;
    if (D != 128) return SPARK_EUNSUPPORTED;
    if (!mask || !chan_energy || !r || !ws) return SPARK_EINVAL;
    if (recovery == SPARK_F_MEAN_RETAINED && T > 0 && !k_packed) return SPARK_EINVAL;
    if (recovery >= SPARK_F_SCORE_MEAN_PRUNED && !k_dense) return SPARK_EINVAL;
    if (!aligned(mask, 16) || !aligned(chan_energy, 16) || !aligned(r, 16) || (cnt && !aligned(cnt, 16)) ||
        (k_packed && !aligned(k_packed, 16)) || (k_dense && !aligned(k_dense, 16)) || !aligned(ws, 256))
        return SPARK_EALIGN;
    const PrefillWs w = prefill_layout(ws, B, S, N_kv);
    if (ws_bytes < w.bytes) return SPARK_ENOSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int BH = B * N_kv;
    hipLaunchKernelGGL(stats_partial_kernel, dim3(w.nblk, BH), dim3(256), 0, st,
                       static_cast<const uint16_t*>(k_packed), mask, static_cast<const uint16_t*>(k_dense),
                       chan_energy, w.sum, w.cnt, w.pruned, S, T, w.nblk, recovery);
    hipLaunchKernelGGL(stats_reduce_kernel, dim3(BH, STATS_CH_BLOCKS), dim3(STATS_THREADS), 0, st,
                       w.sum, w.cnt, w.pruned, chan_energy, r, cnt, S, T, w.nblk, recovery, f_const, 0);
    return hip_status(hipGetLastError());
}

}  // extern "C"

namespace {

// Checks, workspace carving and launch shared by both decode entry points.
// sampled = 0: the fixed recovery vector r; else the sampled F of that mode,
// with r = (mu, sigma, ...) and the channel energy A.
// Packed V (V channels pruned): vp.mask != nullptr.
struct PackedV {
    const void* packed;
    const uint32_t* mask;     // per-entry V pruning
    const float* r;
    float lambda;
    const uint16_t* bmask;    // V pruned in 8-channel blocks (mask unused)
};

int decode_call(const void* q, const void* k_packed, const uint32_t* mask, const void* v, const float* r,
                const float* A, int sampled, uint64_t seed, int B, int S, int N_q, int N_kv, int D, float lambda,
                float scale, int splits, float* out, void* ws, size_t ws_bytes, void* stream,
                const PackedV* vp = nullptr, const int32_t* row_off = nullptr, int S_cap = 0) {
    if (S_cap == 0) S_cap = S;
    if (B < 1 || S < 1 || D < 1 || splits < 0 || S_cap < S) return SPARK_EINVAL;
    // V rows are addressed with 32-bit byte offsets within a head
    if (S_cap >= (1 << 24)) return SPARK_EUNSUPPORTED;
    const int T = kept_or_neg(D, lambda);
    if (T < 0) return SPARK_EINVAL;
    const bool vblocks = vp && vp->bmask;
    const int Tv = vp ? (vblocks ? spark_num_kept_vblocks(D, vp->lambda) : kept_or_neg(D, vp->lambda)) : -1;
    if (vp && Tv < 0) return SPARK_EINVAL;
    if (!(scale == scale)) return SPARK_EINVAL;
    if (int e = check_group(N_q, N_kv)) return e;
    if (D != 128) return SPARK_EUNSUPPORTED;
    const int BH = B * N_kv;
    if ((size_t)BH > (SPARK_DECODE_COUNTER_BYTES / 4)) return SPARK_EUNSUPPORTED;
    if (!q || !mask || !r || !out || !ws || (T > 0 && !k_packed) || (sampled && !A)) return SPARK_EINVAL;
    if (vp ? ((!vp->mask && !vblocks) || !vp->r || (Tv > 0 && !vp->packed)) : !v) return SPARK_EINVAL;
    if (!aligned(q, 16) || !aligned(mask, 16) || (v && !aligned(v, 16)) || !aligned(r, 16) || !aligned(out, 16) ||
        (k_packed && !aligned(k_packed, 16)) || (A && !aligned(A, 16)) || !aligned(ws, 256))
        return SPARK_EALIGN;
    if (vp && ((vp->mask && !aligned(vp->mask, 16)) || (vblocks && !aligned(vp->bmask, 16)) || !aligned(vp->r, 16) ||
               (vp->packed && !aligned(vp->packed, 16))))
        return SPARK_EALIGN;
    const int G = N_q / N_kv;
    int nsplit, chunk;
    // the fast kernel (8 waves, one block per CU) aims for 256 blocks; the
    // generic kernel (4 waves) for 512, two per CU, when two fit in LDS
    const bool ragged = row_off != nullptr;
    const bool generic = (vp && !vblocks) || (ragged ? !decode_fast_ragged_supported(G, S)
                                                      : !decode_fast_supported(G, T, sampled, (size_t)BH * S_cap * T));
    const int waves = generic ? DECODE_THREADS / 64 : DECODE_FAST_THREADS / 64;
    decode_plan(BH, S, splits, &nsplit, &chunk, generic ? DECODE_GENERIC_BLOCKS : 256, waves);
    if (generic && splits == 0 &&
        decode_layout(G, T, nsplit, sampled != 0, vblocks ? -1 : Tv, ragged).lds_bytes > DECODE_LDS_PER_CU / 2)
        decode_plan(BH, S, splits, &nsplit, &chunk, 256, waves);
    if (ws_bytes < decode_ws_bytes(BH, G, nsplit)) return SPARK_ENOSPACE;

    char* base = static_cast<char*>(ws);
    DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.packed = static_cast<const uint16_t*>(k_packed);
    a.mask = mask;
    a.v = static_cast<const uint16_t*>(v);
    a.r = r;
    a.A = A;
    if (vblocks) {
        a.v_packed = static_cast<const uint16_t*>(vp->packed);
        a.v_bmask = vp->bmask;
        a.rv = vp->r;
        a.v_packed_mode = 2;
        a.nbv = Tv;
    } else if (vp) {
        a.v_packed = static_cast<const uint16_t*>(vp->packed);
        a.v_mask = vp->mask;
        a.rv = vp->r;
        a.v_packed_elems = (size_t)BH * S_cap * Tv;
        a.v_packed_mode = 1;
        a.Tv = Tv;
    }
    a.out = out;
    a.counters = reinterpret_cast<uint32_t*>(base);
    a.part_ml = reinterpret_cast<float*>(base + SPARK_DECODE_COUNTER_BYTES);
    a.part_acc = reinterpret_cast<float*>(base + SPARK_DECODE_COUNTER_BYTES +
                                          round_up((size_t)BH * nsplit * 2 * G * sizeof(float), 256));
    a.packed_elems = (size_t)BH * S_cap * (ragged ? 128 : T);
    a.S_cap = S_cap;
    a.row_off = row_off;
    a.S = S;
    a.T = T;
    a.N_q = N_q;
    a.N_kv = N_kv;
    a.nsplit = nsplit;
    a.chunk = chunk;
    const float sc = scale > 0.f ? scale : (float)(1.0 / sqrt((double)D));
    a.qscale = sc * 1.4426950408889634f;
    a.sampled = sampled;
    a.seed_lo = (uint32_t)seed;
    a.seed_hi = (uint32_t)(seed >> 32);
    a.lay = decode_layout(G, T, nsplit, sampled != 0, vblocks ? -1 : Tv, ragged);
    return hip_status(launch_decode(a, G, BH, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int spark_decode_attn(const void* q, const void* k_packed, const uint32_t* mask, const void* v, const float* r,
                      int B, int S, int N_q, int N_kv, int D, float lambda, float scale, int splits,
                      float* out, void* ws, size_t ws_bytes, void* stream) {
    return decode_call(q, k_packed, mask, v, r, nullptr, 0, 0, B, S, N_q, N_kv, D, lambda, scale, splits, out, ws,
                       ws_bytes, stream);
}

int spark_decode_attn_cap(const void* q, const void* k_packed, const uint32_t* mask, const void* v, const float* r,
                          int B, int S, int S_cap, int N_q, int N_kv, int D, float lambda, float scale, int splits,
                          float* out, void* ws, size_t ws_bytes, void* stream) {
    return decode_call(q, k_packed, mask, v, r, nullptr, 0, 0, B, S, N_q, N_kv, D, lambda, scale, splits, out, ws,
                       ws_bytes, stream, nullptr, nullptr, S_cap);
}

int spark_decode_attn_ragged(const void* q, const void* k_packed, const int32_t* row_off, const uint32_t* mask,
                             const void* v, const float* r, int B, int S, int N_q, int N_kv, int D, float scale,
                             int splits, float* out, void* ws, size_t ws_bytes, void* stream) {
    if (!k_packed || !row_off) return SPARK_EINVAL;
    if (!aligned(row_off, 4)) return SPARK_EALIGN;
    if ((size_t)S * 128 > (size_t)INT32_MAX) return SPARK_EUNSUPPORTED;
    return decode_call(q, k_packed, mask, v, r, nullptr, 0, 0, B, S, N_q, N_kv, D, 0.0f, scale, splits, out, ws,
                       ws_bytes, stream, nullptr, row_off);
}

int spark_decode_attn_kv(const void* q, const void* k_packed, const uint32_t* k_mask, const float* r,
                         const void* v_packed, const uint32_t* v_mask, const float* r_v, int B, int S, int N_q,
                         int N_kv, int D, float lambda, float lambda_v, float scale, int splits, float* out, void* ws,
                         size_t ws_bytes, void* stream) {
    if (!v_mask) return SPARK_EINVAL;
    const PackedV vp{v_packed, v_mask, r_v, lambda_v, nullptr};
    return decode_call(q, k_packed, k_mask, nullptr, r, nullptr, 0, 0, B, S, N_q, N_kv, D, lambda, scale, splits, out,
                       ws, ws_bytes, stream, &vp);
}

int spark_decode_attn_kvb(const void* q, const void* k_packed, const uint32_t* k_mask, const float* r,
                          const void* v_packed, const uint16_t* v_bmask, const float* r_v, int B, int S, int N_q,
                          int N_kv, int D, float lambda, float lambda_v, float scale, int splits, float* out, void* ws,
                          size_t ws_bytes, void* stream) {
    if (!v_bmask) return SPARK_EINVAL;
    const PackedV vp{v_packed, nullptr, r_v, lambda_v, v_bmask};
    return decode_call(q, k_packed, k_mask, nullptr, r, nullptr, 0, 0, B, S, N_q, N_kv, D, lambda, scale, splits, out,
                       ws, ws_bytes, stream, &vp);
}

int spark_decode_attn_sampled(const void* q, const void* k_packed, const uint32_t* mask, const void* v,
                              const float* chan_energy, const float* r, int recovery, uint64_t seed,
                              int B, int S, int N_q, int N_kv, int D, float lambda, float scale, int splits,
                              float* out, void* ws, size_t ws_bytes, void* stream) {
    if (recovery != SPARK_F_GAUSSIAN && recovery != SPARK_F_EXPONENTIAL) return SPARK_EINVAL;
    if (!chan_energy) return SPARK_EINVAL;
    return decode_call(q, k_packed, mask, v, r, chan_energy, recovery, seed, B, S, N_q, N_kv, D, lambda, scale,
                       splits, out, ws, ws_bytes, stream);
}

int spark_decode_ws_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws) return SPARK_EINVAL;
    if (!aligned(ws, 256)) return SPARK_EALIGN;
    if (ws_bytes < SPARK_DECODE_COUNTER_BYTES) return SPARK_ENOSPACE;
    const size_t n = SPARK_DECODE_COUNTER_BYTES / 4;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint32_t*>(ws), 0u, n);
    return hip_status(hipGetLastError());
}

}  // extern "C"

namespace {

// Fixed scratch of the allocation-free decode: completion counters, then the
// split partials, laid out as a decode workspace. In host code `scratch` is
// only a symbol: its device address is resolved once per device with
// hipGetSymbolAddress, and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[SPARK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch; on the first call on a
// device, also zero its counters with a fill kernel on `stream`.
int scratch_for_current_device(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPARK_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPARK_EHIP;
        const size_t n = SPARK_DECODE_COUNTER_BYTES / 4;
        hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           static_cast<uint32_t*>(p), 0u, n);
        if (hipGetLastError() != hipSuccess) return SPARK_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SPARK_OK;
}

}  // namespace

extern "C" {

int spark_decode_attn_noalloc(const void* q, const void* k_packed, const uint32_t* mask, const void* v,
                              const float* r, int B, int S, int N_q, int N_kv, int D, float lambda, float scale,
                              int splits, float* out, void* stream) {
    // size check first: nothing is touched for a problem that does not fit
    const size_t need = spark_decode_workspace_bytes(B, S, N_q, N_kv, D, splits);
    if (need == 0) return SPARK_EINVAL;
    if (need > (size_t)SPARK_NOALLOC_SCRATCH_BYTES) return SPARK_ESCRATCH;
    void* ws = nullptr;
    if (int e = scratch_for_current_device(static_cast<hipStream_t>(stream), &ws)) return e;
    const int st = decode_call(q, k_packed, mask, v, r, nullptr, 0, 0, B, S, N_q, N_kv, D, lambda, scale, splits,
                               out, ws, SPARK_NOALLOC_SCRATCH_BYTES, stream);
    return st == SPARK_ENOSPACE ? SPARK_ESCRATCH : st;
}

// window eviction workspace: chunk (m, l) partials, per-row (M, 1/L), scores
static size_t evict_ws_bytes(int BH, int S) {
    return round_up(evict_part_floats(BH, S) * sizeof(float), 256) +
           round_up((size_t)BH * EVICT_MAX_ROWS * 2 * sizeof(float), 256) + round_up((size_t)BH * S * sizeof(float), 256);
}

size_t spark_window_evict_workspace_bytes(int B, int S, int N_q, int N_kv, int D, int window) {
    if (B < 1 || S < 1 || N_kv < 1 || N_q < 1 || D < 1 || window < 1 || N_q % N_kv) return 0;
    return evict_ws_bytes(B * N_kv, S);
}

int spark_window_evict(const void* q_win, const void* k, const void* v, int B, int S, int N_q, int N_kv, int D,
                       int window, int keep, int32_t* idx, void* k_out, void* v_out, float* scores, void* ws,
                       size_t ws_bytes, void* stream) {
    if (B < 1 || S < 1 || D < 1 || window < 1 || window > S || keep < 1 || keep > S) return SPARK_EINVAL;
    if (int e = check_group(N_q, N_kv)) return e;
    if (D != 128) return SPARK_EUNSUPPORTED;
    const int G = N_q / N_kv;
    if ((long)G * window > EVICT_MAX_ROWS || S > EVICT_MAX_S_LONG) return SPARK_EUNSUPPORTED;
    if (!q_win || !k || !idx || !ws || ((k_out == nullptr) != (v_out == nullptr)) || (k_out && !v)) return SPARK_EINVAL;
    if (!aligned(q_win, 16) || !aligned(k, 16) || (v && !aligned(v, 16)) || !aligned(idx, 4) ||
        (k_out && (!aligned(k_out, 16) || !aligned(v_out, 16))) || (scores && !aligned(scores, 4)) || !aligned(ws, 256))
        return SPARK_EALIGN;
    const int BH = B * N_kv;
    if (ws_bytes < evict_ws_bytes(BH, S)) return SPARK_ENOSPACE;
    char* base = static_cast<char*>(ws);
    EvictArgs a{};
    a.q_win = static_cast<const uint16_t*>(q_win);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.idx = idx;
    a.k_out = static_cast<uint16_t*>(k_out);
    a.v_out = static_cast<uint16_t*>(v_out);
    a.part = reinterpret_cast<float*>(base);
    base += round_up(evict_part_floats(BH, S) * sizeof(float), 256);
    a.rowstat = reinterpret_cast<float*>(base);
    base += round_up((size_t)BH * EVICT_MAX_ROWS * 2 * sizeof(float), 256);
    a.scores = scores ? scores : reinterpret_cast<float*>(base);
    a.BH = BH;
    a.S = S;
    a.N_q = N_q;
    a.N_kv = N_kv;
    a.W = window;
    a.R = G * window;
    a.keep = keep;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
    return hip_status(launch_evict(a, static_cast<hipStream_t>(stream)));
}

int spark_read_stream(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream) {
    if (!src || !sink || blocks < 1 || blocks > 65535) return SPARK_EINVAL;
    if (!aligned(src, 16) || (bytes & 15)) return SPARK_EALIGN;
    return hip_status(launch_read_stream(src, bytes, sink, blocks, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
