/*
 * spark.h - C ABI of libspark.so: SparK query-aware, recoverable KV-cache
 * channel pruning (prefill prune, statistics, decode attention) on MI355X.
 *
 * Sources. "KV Cache 还能再砍一刀：SparK 在通道维度上做了一件被忽略多年的事"
 * (ai-paper-analysis.pages.dev walkthrough of arXiv 2508.15212), called "the
 * walkthrough" below, and the AMD blog page "AAAI 2026 AMD论文Spark方法揭秘"
 * (bqwf.cn), called "the blog". Problem size symbols follow the walkthrough's
 * section 1 (B batch, S sequence length, N heads, D head dimension).
 *
 * Conventions for every entry point
 *  - Tensors are dense, row-major, in device memory, and owned by the caller.
 *    The library never allocates, frees or caches device memory; scratch
 *    space comes from the caller's workspace `ws` of `ws_bytes` bytes, sized
 *    by the matching *_workspace_bytes() call (the one exception is the fixed
 *    per-device array of spark_decode_attn_noalloc, part of the library's
 *    code object). Workspaces must be 256-byte
 *    aligned; every tensor pointer must be 16-byte aligned.
 *  - bf16 tensors are passed as `const void*` holding IEEE bfloat16 values.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream). Calls are
 *    asynchronous on that stream and never synchronise with the host.
 *  - Return value: SPARK_OK, or a negative spark_status. Arguments are
 *    checked on the host before anything is launched; on a check failure
 *    nothing is launched and no output is touched. A failed kernel launch
 *    returns SPARK_EHIP. No exception crosses the ABI.
 *  - Only D = 128 is implemented (SPARK_EUNSUPPORTED otherwise) and
 *    G = N_q / N_kv must be 1, 2, 4 or 8 (GQA: query head i reads KV head
 *    i / G). Non-finite inputs give undefined (but memory-safe) results.
 *  - Two calls that share a workspace must not overlap in time.
 */
#ifndef SPARK_H
#define SPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPARK_OK = 0,
    SPARK_EINVAL = -1,        /* bad size, ratio, mode or null pointer */
    SPARK_EUNSUPPORTED = -2,  /* valid but not implemented (D != 128, G not in {1,2,4,8}) */
    SPARK_EALIGN = -3,        /* pointer misaligned */
    SPARK_ENOSPACE = -4,      /* workspace too small */
    SPARK_EHIP = -5,          /* HIP runtime error at launch */
    SPARK_ESCRATCH = -6       /* problem too large for the fixed scratch of spark_decode_attn_noalloc */
} spark_status;

/* Recovery function F for pruned channels (walkthrough section 3.3, F table,
 * and the zero / small-constant fills it compares against). */
typedef enum {
    SPARK_F_MEAN_RETAINED = 0,     /* r_j = mean of retained k_tj over tokens t keeping channel j */
    SPARK_F_ZERO = 1,              /* r_j = 0 */
    SPARK_F_CONST = 2,             /* r_j = f_const */
    SPARK_F_SCORE_MEAN_PRUNED = 3, /* Degenerate F: mu = mean over pruned (t,j) of a_j |k_tj|,
                                      a_j = sqrt(A_j); r_j = mu / a_j (0 if a_j = 0) */
    SPARK_F_GAUSSIAN = 4,          /* sampled F, Gaussian row of the F table: r[0] = mu, r[1] = sigma
                                      (population) of the pruned a_j |k_tj|, r[2..] = 0; decode with
                                      spark_decode_attn_sampled */
    SPARK_F_EXPONENTIAL = 5        /* sampled F, Exponential row (mean mu): r as for SPARK_F_GAUSSIAN */
} spark_recovery;

/* How the window queries form the channel energy A_j = ||q^j||_2^2. */
typedef enum {
    SPARK_QAGG_L2 = 0,   /* A_j = sum over the G*W stacked window rows of q^2 (fp32, sequential) */
    SPARK_QAGG_MEAN = 1  /* A_j = m_j^2, m_j = fp32 sequential sum of the rows (walkthrough
                            section 3.2 mean query; the constant 1/(GW) is dropped) */
} spark_qagg;

/* T = floor((1 - lambda) * D + 0.5), evaluated in double from the fp32
 * lambda: the number of key channels each token keeps (walkthrough section
 * 3.1, the T of the reduced objective; lambda is the pruned fraction, blog
 * Table 1 caption). Returns -1 if lambda is outside [0, 1] or D < 1. */
int spark_num_kept(int D, float lambda);

/* SparK-g (walkthrough section 5.2): T = sum over the ngroups equal channel
 * groups of floor((1 - ratios[i]) * D / ngroups + 0.5). Returns -1 if
 * ngroups is outside 1..8, does not divide D, or a ratio is outside [0, 1]. */
int spark_num_kept_grouped(int D, int ngroups, const float* ratios);

/* Human-readable name of a spark_status. Never NULL. */
const char* spark_strerror(int status);

/* Workspace sizes in bytes (0 on invalid sizes). The prefill size serves
 * spark_prefill_prune, spark_prefill_prune_v and spark_stats; the decode size
 * serves every decode entry point. */
size_t spark_prefill_workspace_bytes(int B, int S, int N_kv, int D);
size_t spark_decode_workspace_bytes(int B, int S, int N_q, int N_kv, int D, int splits);

/*
 * Prefill pruning: channel energy, saliency, per-token top-T, packing and
 * recovery statistics in one call (walkthrough sections 3.1-3.3, Fig. 3
 * prefill half; blog Fig. 2).
 *
 *  q_win        bf16 [B][N_q][W][D]  the last W = window prompt queries
 *  k            bf16 [B][N_kv][S][D] keys
 *  lambda       pruned fraction of channels, in [0, 1]; T = spark_num_kept(D, lambda)
 *  window       W, 1 <= W
 *  qagg         spark_qagg
 *  recovery     spark_recovery; f_const is used by SPARK_F_CONST only
 * Outputs (caller-allocated, fully overwritten):
 *  k_packed     bf16 [B][N_kv][S][T]  retained values, ascending channel order
 *  mask         uint32 [B][N_kv][S][D/32]  bit b of word w set <=> channel 32w+b kept;
 *               exactly T bits set per token. Selection order: saliency key
 *               fl32(A_j * fl32(k_tj^2)) descending, ties to the lower channel.
 *  chan_energy  fp32 [B][N_kv][D]  A_j
 *  r            fp32 [B][N_kv][D]  recovery vector per recovery mode
 *  cnt          int32 [B][N_kv][D] tokens keeping channel j (may be NULL)
 * k_packed may be NULL only when T = 0.
 */
int spark_prefill_prune(const void* q_win, const void* k,
                        int B, int S, int N_q, int N_kv, int D, float lambda, int window,
                        int qagg, int recovery, float f_const,
                        void* k_packed, uint32_t* mask, float* chan_energy, float* r, int32_t* cnt,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * SparK-p prefill pruning (walkthrough section 5.2: per token, the fewest
 * channels whose cumulative saliency reaches p of the token's total). With
 * key_tj as in spark_prefill_prune, w_tj = fl32(sqrt(key_tj)) (correctly
 * rounded) and every sum over a token's D = 128 channels taken as the fp32
 * pairwise tree that adds channel j + 64 to j, then j + 32, ..., j + 1:
 * target = fl32(p * sum of all w); theta = the largest key value whose sum
 * of w over {key >= theta} reaches the target; the token keeps the channels
 * with key >= theta (ties at theta kept together; none if all w are 0).
 *  p          in (0, 1] (the page uses 0.99), fp32
 * Outputs (caller-allocated):
 *  k_packed   bf16 [B][N_kv][S * D]: each head's region holds its tokens'
 *             kept values back to back, token t at [row_off[t], row_off[t+1])
 *             (ascending channel); the rest of the region is not written
 *  row_off    int32 [B][N_kv][S + 1]: row offsets within the head's region,
 *             row_off[0] = 0, row_off[S] = the head's kept total
 *  mask, chan_energy, r, cnt   as for spark_prefill_prune (r for every
 *             recovery mode; the pruned count of the score means is
 *             S * D minus the kept total)
 * Workspace: spark_prefill_workspace_bytes. Requires S * D < 2^31.
 */
int spark_prefill_prune_topp(const void* q_win, const void* k, int B, int S, int N_q, int N_kv, int D, float p,
                             int window, int qagg, int recovery, float f_const, void* k_packed, int32_t* row_off,
                             uint32_t* mask, float* chan_energy, float* r, int32_t* cnt, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * SparK-g prefill pruning (walkthrough section 5.2: channels grouped by
 * importance, each group pruned at its own ratio, the least important
 * hardest). Per (b, KV head) the channels are ranked by the channel energy
 * A_j (descending, ties to the lower channel) and cut into ngroups equal
 * groups; group i (0 = most important) keeps, for every token, its
 * floor((1 - ratios[i]) * D / ngroups + 0.5) members of largest saliency key
 * (ties to the lower channel). Every token keeps the same
 * T = spark_num_kept_grouped(D, ngroups, ratios) channels, so the outputs
 * have the layouts of spark_prefill_prune with that T, and decode runs
 * through spark_decode_attn with lambda = 1 - T / D.
 *  ngroups, ratios   1..8 groups dividing D; ratios: host array of ngroups
 *                    pruned fractions in [0, 1] (the page's g = 4 uses
 *                    0.25, 0.5, 0.75, 1.0)
 * Other arguments, outputs and return codes as for spark_prefill_prune.
 */
int spark_prefill_prune_grouped(const void* q_win, const void* k, int B, int S, int N_q, int N_kv, int D,
                                int ngroups, const float* ratios, int window, int qagg, int recovery, float f_const,
                                void* k_packed, uint32_t* mask, float* chan_energy, float* r, int32_t* cnt,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * Decode-time cache growth. The pages prune only at prefill; the reading
 * here: a cache is allocated with a capacity of S_cap tokens per (b, KV
 * head), each generated token's key is pruned with the prefill's channel
 * energy by the same rule as the prompt's keys and appended, its V row is
 * appended dense, and r stays as the prefill computed it.
 *
 * spark_prefill_prune_cap: spark_prefill_prune writing k_packed
 * [B][N_kv][S_cap][T] and mask [B][N_kv][S_cap][D/32] (rows S..S_cap-1 left
 * untouched); S <= S_cap.
 */
int spark_prefill_prune_cap(const void* q_win, const void* k, int B, int S, int S_cap, int N_q, int N_kv, int D,
                            float lambda, int window, int qagg, int recovery, float f_const,
                            void* k_packed, uint32_t* mask, float* chan_energy, float* r, int32_t* cnt,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Append one token per (b, KV head) at row pos (0 <= pos < S_cap):
 *  k_new, v_new  bf16 [B][N_kv][D]  the new token's key and value
 *  chan_energy   fp32 [B][N_kv][D]  A_j from the prefill
 * Writes mask[b][h][pos], k_packed[b][h][pos][0..T) (T = spark_num_kept(D,
 * lambda); key fl32(A_j k_j^2), top-T, ties to the lower channel) and
 * v[b][h][pos] (bf16 [B][N_kv][S_cap][D]). Other rows are untouched.
 */
int spark_append_token(const void* k_new, const void* v_new, const float* chan_energy, int B, int N_kv, int D,
                       float lambda, int pos, int S_cap, void* k_packed, uint32_t* mask, void* v, void* stream);

/*
 * Recovery statistics recomputed from a stored pruned cache (walkthrough
 * section 3.3 step 1), e.g. to switch F without pruning again.
 *  k_packed, mask, chan_energy   as written by spark_prefill_prune
 *  k_dense      bf16 [B][N_kv][S][D]; required by SPARK_F_SCORE_MEAN_PRUNED and
 *               the sampled F (the pruned values are not in the packed store),
 *               else ignored
 *  r, cnt       outputs as in spark_prefill_prune (cnt may be NULL)
 */
int spark_stats(const void* k_packed, const uint32_t* mask, const float* chan_energy,
                const void* k_dense, int B, int S, int N_kv, int D, float lambda,
                int recovery, float f_const, float* r, int32_t* cnt,
                void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step over the pruned cache: each pruned channel of each cached
 * key takes r_j, then ordinary softmax attention runs over all S tokens with
 * dense V (walkthrough section 3.3 and Fig. 3 decode half; blog Fig. 2).
 *  q        bf16 [B][N_q][D]  one new query per head
 *  k_packed, mask, r         the pruned cache (layouts as above)
 *  v        bf16 [B][N_kv][S][D]
 *  scale    softmax scale; <= 0 selects 1/sqrt(D)
 *  splits   sequence splits per (b, KV head); 0 lets the library choose
 *           (about 256 blocks in all for the matrix-core kernel, which takes
 *           every T from 1 to D and every group size; 512 for the generic
 *           one, used for packed V, the sampled F outside G = 4 with T in
 *           {26, 38, 48, 64}, T = 0 and packed caches shorter than one
 *           lane's row request (at most 68 dwords in all), when two blocks
 *           fit in one CU's LDS; never fewer 64-token tiles
 *           per block than its 8 or 4 waves); larger values are clamped to
 *           min(256, ceil(S / 64))
 *  out      fp32 [B][N_q][D]
 * No causal mask: the query attends to every cached token. fp32 arithmetic
 * on bf16 inputs. The first SPARK_DECODE_COUNTER_BYTES of ws hold completion
 * counters, one per (b, KV head), that must be zero before the first call
 * (spark_decode_ws_init); every call that completes leaves them zero again.
 * B * N_kv above SPARK_DECODE_COUNTER_BYTES / 4 (65536), and 2^24 or more
 * cached tokens per head (the head stride, S or S_cap), are SPARK_EUNSUPPORTED.
 */
#define SPARK_DECODE_COUNTER_BYTES (256u << 10)
int spark_decode_attn(const void* q, const void* k_packed, const uint32_t* mask, const void* v,
                      const float* r, int B, int S, int N_q, int N_kv, int D, float lambda,
                      float scale, int splits, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step with a sampled recovery F (walkthrough section 3.3, steps
 * 2-4 and the Gaussian and Exponential rows of the F table): every pruned
 * channel j of every cached key t draws its own saliency sample w_tj and is
 * back-solved to w_tj / a_j (0 if a_j = 0), a_j = sqrt(A_j); then attention
 * runs as in spark_decode_attn.
 *  chan_energy  fp32 [B][N_kv][D]  A_j, as written by spark_prefill_prune
 *  r            fp32 [B][N_kv][D]  (mu, sigma, 0, ...) as written for the same recovery
 *  recovery     SPARK_F_GAUSSIAN: w = mu + sigma z, z standard normal;
 *               SPARK_F_EXPONENTIAL: w exponential with mean mu
 *  seed         Philox4x32-10 key (low word, high word). Token t, channel
 *               group jg = j / 4 of (b, KV head h) uses the counter
 *               (t, jg, b * N_kv + h, 0); its four outputs x_i give
 *               u_i = (x_i + 1/2) 2^-32 for channels 4 jg + i. Gaussian: z by
 *               Box-Muller, R = sqrt(-2 ln u_0) with angle 2 pi u_1 giving
 *               z_0 = R cos, z_1 = R sin, and likewise (u_2, u_3) for z_2, z_3.
 *               Exponential: w = -mu ln u_i. The same seed gives the same
 *               samples on every call and every split count.
 * Other arguments, the workspace and the return codes as for
 * spark_decode_attn; SPARK_EINVAL also for another recovery or a NULL
 * chan_energy. Samples are drawn in fp32 (logf, sqrtf, sincospif).
 */
int spark_decode_attn_sampled(const void* q, const void* k_packed, const uint32_t* mask, const void* v,
                              const float* chan_energy, const float* r, int recovery, uint64_t seed,
                              int B, int S, int N_q, int N_kv, int D, float lambda, float scale, int splits,
                              float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * spark_decode_attn over the first S tokens of a cache of capacity S_cap
 * (k_packed [B][N_kv][S_cap][T], mask [B][N_kv][S_cap][D/32], v
 * [B][N_kv][S_cap][D]); S <= S_cap. The workspace size is that of
 * spark_decode_workspace_bytes(B, S, ...).
 */
int spark_decode_attn_cap(const void* q, const void* k_packed, const uint32_t* mask, const void* v, const float* r,
                          int B, int S, int S_cap, int N_q, int N_kv, int D, float lambda, float scale, int splits,
                          float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step over a ragged pruned cache (spark_prefill_prune_topp):
 * as spark_decode_attn with the kept values of token t at
 * [row_off[t], row_off[t + 1]) of its head's region of S * D elements.
 * mask and row_off must agree (the popcount of token t's mask equals
 * row_off[t + 1] - row_off[t]); otherwise results are undefined but every
 * read stays inside the head's region.
 */
int spark_decode_attn_ragged(const void* q, const void* k_packed, const int32_t* row_off, const uint32_t* mask,
                             const void* v, const float* r, int B, int S, int N_q, int N_kv, int D, float scale,
                             int splits, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * V-channel pruning (walkthrough section 4.4: V channels are pruned together
 * with K by a norm-based rule that the page does not spell out; read
 * here as per-token top-T_v of |v_tj|). Same selection, packing and retained-
 * mean statistics as the keys' with every channel energy equal to 1.
 *  v            bf16 [B][N_kv][S][D]
 *  lambda_v     pruned fraction of V channels; T_v = spark_num_kept(D, lambda_v)
 * Outputs (caller-allocated, fully overwritten):
 *  v_packed     bf16 [B][N_kv][S][T_v]  retained values, ascending channel order (NULL only if T_v = 0)
 *  v_mask       uint32 [B][N_kv][S][D/32]  exactly T_v bits per token; order |v| descending
 *               (key fl32(v^2)), ties to the lower channel
 *  r_v          fp32 [B][N_kv][D]  mean of the retained v_tj over the tokens keeping
 *               channel j (0 if none), rounded to the nearest bfloat16 (ties to
 *               even), the precision of the cached entries it stands in for: the
 *               value a pruned V entry takes
 *  cnt          int32 [B][N_kv][D]  tokens keeping channel j (may be NULL)
 * Workspace: spark_prefill_workspace_bytes(B, S, N_kv, D).
 */
int spark_prefill_prune_v(const void* v, int B, int S, int N_kv, int D, float lambda_v, void* v_packed,
                          uint32_t* v_mask, float* r_v, int32_t* cnt, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step over a cache whose K and V channels are both pruned
 * (walkthrough sections 3.3 and 4.4): K_hat as in spark_decode_attn and
 * V_hat = v_mask ? stored value : r_v[j], then softmax attention. V is read
 * from the packed store only (2 T_v + 16 bytes per token and KV head instead
 * of 2 D).
 *  k_packed, k_mask, r        the K cache, as for spark_decode_attn
 *  v_packed, v_mask, r_v      the V cache, as written by spark_prefill_prune_v
 *  lambda, lambda_v           pruned fractions of K and V
 * Other arguments, the workspace and the return codes as for
 * spark_decode_attn (SPARK_EINVAL also for a NULL v_mask or r_v, or a NULL
 * v_packed with T_v > 0).
 */
int spark_decode_attn_kv(const void* q, const void* k_packed, const uint32_t* k_mask, const float* r,
                         const void* v_packed, const uint32_t* v_mask, const float* r_v, int B, int S, int N_q,
                         int N_kv, int D, float lambda, float lambda_v, float scale, int splits, float* out, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * V pruned in blocks of 8 consecutive channels: a second reading of the
 * norm-based V rule of walkthrough section 4.4, under which a token keeps
 * whole blocks: the n_b blocks whose entries have the largest L2 norm,
 * compared squared as an fp32 sum of the block's 8 squares (exact for bf16)
 * added in channel order, ties to the lower block. A block is the 16-byte
 * unit in which decode reads V, so the pruned cache is read with the same
 * requests as a dense one (2 * 8 n_b + 2 bytes per token and KV head
 * instead of 2 D).
 */
#define SPARK_VBLOCK 8

/* n_b = floor((1 - lambda_v) * D / 8 + 0.5) (lambda_v as an IEEE fp32 value)
 * blocks kept per token; -1 if D is not a positive multiple of 8 or lambda_v
 * lies outside [0, 1]. */
int spark_num_kept_vblocks(int D, float lambda_v);

/* Block masks per head for a cache of S (or capacity S_cap) tokens: S
 * rounded up to a multiple of 64 (0 for S < 1). */
size_t spark_vblock_mask_stride(int S);

/*
 * Block-mode V pruning of a V cache.
 *  v            bf16 [B][N_kv][S][D]
 *  lambda_v     pruned fraction of V blocks; n_b = spark_num_kept_vblocks(D, lambda_v)
 * Outputs (caller-allocated, fully overwritten):
 *  v_packed     bf16 [B][N_kv][S][8 n_b]  each token's kept blocks back to back in
 *               ascending block order (NULL only if n_b = 0)
 *  v_bmask      uint16 [B][N_kv][spark_vblock_mask_stride(S)]  per token a 16-bit mask, bit i
 *               for block i (channels 8i .. 8i + 7), exactly n_b bits set. Stored
 *               tile-interleaved: token t of a head at entry
 *               64 floor(t / 64) + 16 (t mod 4) + floor((t mod 64) / 4); the entries
 *               of the last tile past S are written as 0
 *  r_v          fp32 [B][N_kv][D]  mean of v_tj over the tokens keeping channel j's block
 *               (0 if none), rounded to the nearest bfloat16 (ties to even): the value a
 *               pruned V entry takes
 *  cnt          int32 [B][N_kv][D]  tokens keeping channel j's block (may be NULL)
 * Workspace: spark_prefill_workspace_bytes(B, S, N_kv, D).
 * SPARK_EUNSUPPORTED for D != 128 or B * N_kv > 65535.
 */
int spark_prefill_prune_vblocks(const void* v, int B, int S, int N_kv, int D, float lambda_v, void* v_packed,
                                uint16_t* v_bmask, float* r_v, int32_t* cnt, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode step over a cache whose K channels are pruned and whose V is
 * pruned in 8-channel blocks (walkthrough sections 3.3 and 4.4): K_hat as in
 * spark_decode_attn, V_hat = the token's block if kept, else r_v of its
 * channels, then softmax attention.
 *  k_packed, k_mask, r          the K cache, as for spark_decode_attn
 *  v_packed, v_bmask, r_v       the V cache, as written by spark_prefill_prune_vblocks
 *                               (r_v is read as bfloat16: other values are rounded to
 *                               the nearest)
 *  lambda, lambda_v             pruned fractions of K channels and V blocks
 * Other arguments, the workspace and the return codes as for
 * spark_decode_attn (SPARK_EINVAL also for a NULL v_bmask or r_v, or a NULL
 * v_packed with n_b > 0).
 */
int spark_decode_attn_kvb(const void* q, const void* k_packed, const uint32_t* k_mask, const float* r,
                          const void* v_packed, const uint16_t* v_bmask, const float* r_v, int B, int S, int N_q,
                          int N_kv, int D, float lambda, float lambda_v, float scale, int splits, float* out, void* ws,
                          size_t ws_bytes, void* stream);

/* Zero the decode completion counters of a workspace (a fill kernel on
 * `stream`; safe to record in a HIP graph). */
int spark_decode_ws_init(void* ws, size_t ws_bytes, void* stream);

/*
 * spark_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The completion counters and split
 * partials live in a fixed device array of SPARK_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends; the call
 * itself allocates nothing and calls no allocating routine.
 *  Arguments, layouts and results as for spark_decode_attn (same kernels, same
 *  split plan, so the output is bit-identical to spark_decode_attn with the
 *  same splits).
 *  Returns SPARK_ESCRATCH if the problem needs more scratch than the array
 *  holds: spark_decode_workspace_bytes(B, S, N_q, N_kv, D, splits) must not
 *  exceed SPARK_NOALLOC_SCRATCH_BYTES.
 *  The first call on a device resolves the array's address and zeroes its
 *  counters with a fill kernel on `stream`; every completed call leaves them
 *  zero again. All calls on one GPU share the array: calls that overlap in
 *  time on one GPU (different streams, or host threads) race and give
 *  undefined results; serialise them.
 */
#define SPARK_NOALLOC_SCRATCH_BYTES (8u << 20)
int spark_decode_attn_noalloc(const void* q, const void* k_packed, const uint32_t* mask, const void* v,
                              const float* r, int B, int S, int N_q, int N_kv, int D, float lambda, float scale,
                              int splits, float* out, void* stream);

/*
 * Observation-window token eviction (SnapKV style), the stage SparK is
 * stacked on in the pages' combination with eviction (walkthrough section
 * 4.1; section 3.2 borrows the observation window). Not SparK itself.
 * Per (b, KV head h): the G*W window queries q_win[b][hG+g][w] sit at
 * positions S-W+w and see tokens t <= S-W+w; each row's softmax of
 * q.k_t / sqrt(D) over those tokens is summed over the G*W rows into
 * score[t]; the `keep` highest-scoring tokens (ties to the lower t) are kept.
 *  q_win    bf16 [B][N_q][W][D]
 *  k, v     bf16 [B][N_kv][S][D]
 *  idx      int32 [B][N_kv][keep]  kept token indices, ascending
 *  k_out, v_out  bf16 [B][N_kv][keep][D]  gathered rows; both NULL skips
 *           the gather
 *  scores   fp32 [B][N_kv][S]  window-summed scores (NULL: kept in ws)
 * Logits run on the matrix cores (bf16 inputs, fp32 accumulation); two
 * passes over K. Requires D = 128, G*W <= 128 and S <= 1048576 (else
 * SPARK_EUNSUPPORTED),
 * 1 <= W <= S, 1 <= keep <= S (else SPARK_EINVAL). Scores that tie exactly in
 * fp32 are broken by the lower t; scores are fp32, so tokens whose scores
 * differ by less than their rounding error may be ordered either way.
 */
size_t spark_window_evict_workspace_bytes(int B, int S, int N_q, int N_kv, int D, int window);
int spark_window_evict(const void* q_win, const void* k, const void* v, int B, int S, int N_q, int N_kv,
                       int D, int window, int keep, int32_t* idx, void* k_out, void* v_out, float* scores,
                       void* ws, size_t ws_bytes, void* stream);

/* Diagnostic, not part of SparK: read `bytes` (a multiple of 16, 16-byte
 * aligned) from device memory with `blocks` x 256 threads, folding the data
 * into sink[0 .. blocks-1] (uint32, XOR-accumulated). Used to measure the
 * practical HBM read bandwidth that decode is compared with. */
int spark_read_stream(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARK_H */
