// Kernel declarations and launch constants of libspark (internal header).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PRUNE_TOKENS_PER_BLOCK 64
#define CHAN_ENERGY_ROWS 128
// stats reduction: per (b, kv head) STATS_CH_BLOCKS blocks of 128 / STATS_CH_BLOCKS channels,
// each channel summed over STATS_PARTS ranges of block partials
#define STATS_CH_BLOCKS 4
#define STATS_PARTS 32
#define STATS_THREADS 1024
#define DECODE_THREADS 256
#define DECODE_FAST_THREADS 512
// LDS of the exact-T matrix-core decode kernels: q' and r tables with a flag
// slot (4112 B), then per wave the slot list of the largest T (64 lanes x 68
// u16) and 1 KiB of p
#define DECODE_FAST_LDS_BYTES (4112 + (DECODE_FAST_THREADS / 64) * (8704 + 1024))
#define DECODE_TILE 64
#define DECODE_MAX_SPLITS 256
#define DECODE_RAGGED_CHUNKS (DECODE_TILE * 128 * 2 / 16 + 1)   // 16-byte chunks of a tile of full rows, + misalignment
#define DECODE_GENERIC_BLOCKS 512    // blocks the generic decode kernel aims for when splits = 0
#define DECODE_LDS_PER_CU (160 * 1024)
// window eviction: at most 128 stacked window rows (G * W), tokens per block
#define EVICT_MAX_ROWS 128
#define EVICT_WAVE_ROWS 32
#define EVICT_CHUNK 1024
#define EVICT_TILE 64
#define EVICT_SELECT_THREADS 1024
#define EVICT_MAX_S (EVICT_SELECT_THREADS * 64)   // tokens per (b, KV head) the register-held select handles
#define EVICT_MAX_S_LONG (1 << 20)                 // longer caches: the select that re-reads the scores

namespace spark {

__global__ void chan_energy_kernel(const uint16_t* q_win, float* A, int N_q, int N_kv, int W, int qagg);
#define SPARK_MAX_GROUPS 8
// SparK-g: ngroups equal channel groups, each keeping T[i] of its `size` members per token
struct GroupSpec {
    int n;
    int size;
    int T[SPARK_MAX_GROUPS];
};
template <int SEL>
__global__ void select_pack_kernel(const uint16_t* k, const float* A, uint16_t* k_packed, uint32_t* mask,
                                   double* part_sum, int32_t* part_cnt, double* part_pruned,
                                   int S, int T, int nblk, int recovery, const uint8_t* gid, GroupSpec grp,
                                   float top_p, int32_t* tok_cnt, int32_t* blk_cnt, int S_out);
__global__ void append_token_kernel(const uint16_t* k_new, const uint16_t* v_new, const float* A, uint16_t* k_packed,
                                    uint32_t* mask, uint16_t* v, int T, int pos, int S_cap);
__global__ void topp_scan_kernel(int32_t* blk_cnt, int nblk);
__global__ void topp_pack_kernel(const uint16_t* k, const uint32_t* mask, uint16_t* k_packed, int32_t* row_off,
                                 const int32_t* blk_base, int S, int nblk);
__global__ void channel_groups_kernel(const float* A, uint8_t* gid, int ngroups);
__global__ void stats_partial_kernel(const uint16_t* k_packed, const uint32_t* mask, const uint16_t* k_dense,
                                     const float* A, double* part_sum, int32_t* part_cnt, double* part_pruned,
                                     int S, int T, int nblk, int recovery);
__global__ void stats_reduce_kernel(const double* part_sum, const int32_t* part_cnt, const double* part_pruned,
                                    const float* A, float* r, int32_t* cnt, int S, int T, int nblk,
                                    int recovery, float f_const, int round_bf16);
__global__ void fill_u32_kernel(uint32_t* p, uint32_t value, size_t n);
// V pruned in 8-channel blocks: 16-bit block masks per token, stored
// tile-interleaved so that a decode lane reading rows 4i + tau of a 64-token
// tile finds its 16 masks in 32 contiguous bytes; a head holds its capacity
// rounded up to whole tiles
__host__ __device__ constexpr size_t vblock_mask_stride(int S_cap) {
    return ((size_t)S_cap + DECODE_TILE - 1) / DECODE_TILE * DECODE_TILE;
}
__host__ __device__ constexpr uint32_t vblock_mask_index(int t) {
    return (uint32_t)(t & ~(DECODE_TILE - 1)) + 16u * (uint32_t)(t & 3) + (uint32_t)((t & (DECODE_TILE - 1)) >> 2);
}
__global__ void vblock_select_kernel(const uint16_t* v, uint16_t* v_packed, uint16_t* bmask, double* part_sum,
                                     int32_t* part_cnt, int S, int nb, int nblk, int S_cap);

// LDS layout of the decode kernel (computed on the host for T and G).
struct DecodeLayout {
    uint32_t tab_stride;   // bytes per channel entry of the q'/r table: G floats of q', then r
    uint32_t row_bytes;    // LDS bytes between staged packed rows of consecutive tokens
    uint32_t padded;       // 1: rows padded to an odd dword count (T/2 even), staged dword by dword
    uint32_t half_T;       // T / 2 (padded rows)
    uint32_t magic;        // ceil(2^32 / half_T): u / half_T == umulhi(u, magic) for u < 2^16
    uint32_t list_bytes;   // per wave: kept-channel table offsets, u16 [T][64]
    uint32_t stage_bytes;  // per wave: staged packed rows of one 64-token tile
    uint32_t ptab_bytes;   // per wave: p of the tile, [64][G] fp32
    uint32_t vstage_bytes; // per wave, packed V only: staged packed V rows of one tile (+ slack)
    uint32_t vmask_bytes;  // per wave, packed V only: the tile's V masks, [64] x 16 B
    uint32_t kv_bytes;     // per wave: max(list + stage, vstage + vmask) (packed V reuses the key region)
    uint32_t wave_bytes;   // kv + ptab
    uint32_t tab_bytes;    // 128 * tab_stride, plus the [128][G] fp32 q' ns table of the sampled F
    uint32_t lds_bytes;    // whole block (dynamic LDS)
};

struct DecodeArgs {
    const uint16_t* q;        // [B][N_q][128]
    const uint16_t* packed;   // [B][N_kv][S][T]
    const uint32_t* mask;     // [B][N_kv][S][4]
    const uint16_t* v;        // [B][N_kv][S][128]
    const float* r;           // [B][N_kv][128]; sampled F: (mu, sigma) in entries 0, 1
    const float* A;           // [B][N_kv][128] channel energy (sampled F only)
    const uint16_t* v_packed; // [B][N_kv][S][Tv] (V channels pruned only)
    const uint32_t* v_mask;   // [B][N_kv][S][4]
    const float* rv;          // [B][N_kv][128] recovery of pruned V entries
    const uint16_t* v_bmask;  // V pruned in 8-channel blocks: [B][N_kv][vblock_mask_stride(S_cap)] block masks
    const int32_t* row_off;   // ragged packed rows (SparK-p): [B][N_kv][S + 1] offsets within a head's
                              // region of S * 128 elements of `packed`; null otherwise
    float* out;               // [B][N_q][128]
    float* part_ml;           // [B*N_kv][nsplit][2][G]
    float* part_acc;          // [B*N_kv][nsplit][G][128]
    uint32_t* counters;       // [B*N_kv]
    size_t packed_elems;      // B*N_kv*S*T
    size_t v_packed_elems;    // B*N_kv*S*Tv
    int S, T, N_q, N_kv, nsplit, chunk;
    int S_cap;                // head stride of packed, mask and v in tokens (>= S; S unless a cache grows)
    float qscale;             // softmax scale * log2(e)
    int sampled;              // 0, or the sampled F (4 Gaussian, 5 Exponential)
    int v_packed_mode;        // 1: V channels pruned (v_packed, v_mask, rv; v unused); 2: V pruned in
                              // 8-channel blocks (v_packed [B][N_kv][S_cap][8 nbv], v_bmask, rv)
    int Tv;                   // V channels kept per token (v_packed_mode 1)
    int nbv;                  // V blocks kept per token (v_packed_mode 2)
    uint32_t seed_lo, seed_hi;  // Philox key of the sampled F
    DecodeLayout lay;
};

struct EvictArgs {
    const uint16_t* q_win;    // [B][N_q][W][128]
    const uint16_t* k;        // [B][N_kv][S][128]
    const uint16_t* v;        // [B][N_kv][S][128]
    int32_t* idx;             // [B][N_kv][keep]
    uint16_t* k_out;          // [B][N_kv][keep][128] or null (then v_out too: no gather)
    uint16_t* v_out;
    float* scores;            // [B][N_kv][S]
    float* part;              // [B*N_kv][nchunk][EVICT_MAX_ROWS][2]
    float* rowstat;           // [B*N_kv][EVICT_MAX_ROWS][2]
    int BH, S, N_q, N_kv, W, R, keep;
    float scale_log2;         // log2(e) / sqrt(D)
};

hipError_t launch_evict(const EvictArgs& a, hipStream_t stream);
size_t evict_part_floats(int BH, int S);

hipError_t launch_read_stream(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream);

// Launch the decode kernel for group size G; returns a hipError_t.
hipError_t launch_decode(const DecodeArgs& a, int G, int BH, hipStream_t stream);
// whether the matrix-core decode kernel takes fixed rows of T for group size
// G (sampled: the sampled F), the packed buffer holding packed_elems values
bool decode_fast_supported(int G, int T, int sampled, size_t packed_elems);
// ragged rows (SparK-p) on the matrix-core kernel
bool decode_fast_ragged_supported(int G, int S);
// Runtime-T variants of the matrix-core kernel: the largest row length of
// T's variant, and the dwords each lane requests for a row (the row's dwords
// plus one when odd rows start mid-dword, in whole 16-byte requests).
constexpr int decode_fast_bucket(int T) { return T <= 32 ? 32 : T <= 64 ? 64 : T <= 96 ? 96 : 128; }
constexpr int decode_fast_kr(int TB, bool odd) { return 4 * ((TB / 2 + (odd ? 1 : 0) + 3) / 4); }
// the same for the exact-T variants: T / 2 for even T (exact loads), else
// whole 16-byte requests covering the row and the dword after it (the funnel
// shift's upper operand for the last slot)
constexpr int decode_fast_kr_exact(int T) { return T % 2 == 0 ? T / 2 : 4 * ((T / 2 + 2 + 3) / 4); }
// whether an exact-T variant exists for (G, T) (sampled: the sampled F)
bool decode_fast_exact(int G, int T, int sampled);
// matrix-core launchers: exact-T variants (G = 4, T in {26, 38, 48, 64},
// fixed or sampled F; more pruning ratios and group sizes with the fixed F)
// and the runtime-T / ragged variants per group size
hipError_t launch_fast_fixed(const DecodeArgs& a, dim3 grid, hipStream_t stream);
hipError_t launch_fast_fixed2(const DecodeArgs& a, int G, dim3 grid, hipStream_t stream);
hipError_t launch_fast_g1(const DecodeArgs& a, dim3 grid, hipStream_t stream);
hipError_t launch_fast_g2(const DecodeArgs& a, dim3 grid, hipStream_t stream);
hipError_t launch_fast_g4(const DecodeArgs& a, dim3 grid, hipStream_t stream);
hipError_t launch_fast_g8(const DecodeArgs& a, dim3 grid, hipStream_t stream);
// block-pruned V: per group size, the runtime-T variants (and at G = 4 the
// exact T = 64 and 26)
hipError_t launch_fast_vb_g1(const DecodeArgs& a, dim3 grid, hipStream_t stream);
hipError_t launch_fast_vb_g2(const DecodeArgs& a, dim3 grid, hipStream_t stream);
hipError_t launch_fast_vb_g4(const DecodeArgs& a, dim3 grid, hipStream_t stream);
hipError_t launch_fast_vb_g8(const DecodeArgs& a, dim3 grid, hipStream_t stream);
DecodeLayout decode_layout(int G, int T, int nsplit, bool sampled, int Tv, bool ragged = false);

}  // namespace spark
