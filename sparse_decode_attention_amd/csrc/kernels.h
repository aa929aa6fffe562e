// Kernel declarations and launch constants of libspark (internal header).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define PRUNE_TOKENS_PER_BLOCK 256
#define DECODE_THREADS 256
#define DECODE_TILE 64

namespace spark {

__global__ void chan_energy_kernel(const uint16_t* q_win, float* A, int N_q, int N_kv, int W, int qagg);
__global__ void select_pack_kernel(const uint16_t* k, const float* A, uint16_t* k_packed, uint32_t* mask,
                                   double* part_sum, int32_t* part_cnt, double* part_pruned,
                                   int S, int T, int nblk, int recovery);
__global__ void stats_partial_kernel(const uint16_t* k_packed, const uint32_t* mask, const uint16_t* k_dense,
                                     const float* A, double* part_sum, int32_t* part_cnt, double* part_pruned,
                                     int S, int T, int nblk, int recovery);
__global__ void stats_reduce_kernel(const double* part_sum, const int32_t* part_cnt, const double* part_pruned,
                                    const float* A, float* r, int32_t* cnt, int S, int T, int nblk,
                                    int recovery, float f_const);
__global__ void fill_u32_kernel(uint32_t* p, uint32_t value, size_t n);

struct DecodeArgs {
    const uint16_t* q;        // [B][N_q][128]
    const uint16_t* packed;   // [B][N_kv][S][T]
    const uint32_t* mask;     // [B][N_kv][S][4]
    const uint16_t* v;        // [B][N_kv][S][128]
    const float* r;           // [B][N_kv][128]
    float* out;               // [B][N_q][128]
    float* part_ml;           // [B*N_kv][nsplit][2][G]
    float* part_acc;          // [B*N_kv][nsplit][G][128]
    uint32_t* counters;       // [B*N_kv]
    size_t packed_elems;      // B*N_kv*S*T
    int S, T, N_q, N_kv, nsplit, chunk;
    float qscale;             // softmax scale * log2(e)
    uint32_t lds_stage_bytes; // per-wave packed staging
};

// Launch the decode kernel for group size G; returns a hipError_t.
hipError_t launch_decode(const DecodeArgs& a, int G, int BH, hipStream_t stream);
size_t decode_lds_bytes(int G, int T);
uint32_t decode_stage_bytes(int T);

}  // namespace spark
