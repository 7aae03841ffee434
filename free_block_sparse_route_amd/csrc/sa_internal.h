// Internal launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16;

constexpr size_t kSelectLdsBudget = 80 * 1024;   // proxy rows of one select workgroup (gfx950: up to 160 KB per workgroup)
constexpr int kMaxKeyBlocks = 16384 - 16;       // n_kb limit: one proxy row at G = 1 stays within 64 KB

struct PoolArgs {
    int N, block_q, block_k, n_qb, n_kb, words;
    int first;                           // first tensor pooled: 0 = Q, K, V; 1 = K, V (select pools Q)
    float *q_mean, *k_mean, *v_mean;
    bf16 *kv_split;                      // [BH][2][words][64][D] hi/lo residual tiles
};

struct SelectArgs {
    int N, block_q, block_k, n_qb, n_kb, mask_words, kv_idx_cap;
    int exact_tile_rows;                 // key rows per exact attention tile (cost model)
    int tau_mode, max_keep, min_keep, n_prefix;
    int stats_only;                      // fused routing pre-pass: row statistics only
    float scale, ln_tau;                 // ln_tau = -inf when tau == 0
    float topp_target;                   // 1 - tau: proxy mass the TOPP mode retains
    const void *q;                       // queries [BH][N][D]: select pools its own query blocks
    int q_bf16;                          // q's element type: 1 = bf16, 0 = fp32
    float *q_mean;                       // written by select (pooled there)
    const float *k_mean;
    int32_t *kv_count, *kv_idx, *cost, *work_order;
    uint32_t *kv_mask;
    float *row_stats;
    const bf16 *kv_split;                // residual tiles written by pool (read for the bounds)
    float *k_bounds;                     // [BH][mask_words][2] key-mean and remainder norm bounds per residual tile
};

struct FlashArgs {
    int N, block_q, block_k, n_qb, n_kb, mask_words, kv_idx_cap;
    int Nq;                              // query rows per (b, h): N, or the probe count of a probe pass
    float *o32;                          // when set, O is written here in fp32 (o unused)
    // dense path only: the key tiles split into kv_splits ranges (>= 1), work
    // item (query block, split s) writing its O and lse at o32 + s * split_o,
    // lse + s * split_l, for a later merge
    int kv_splits;
    size_t split_o, split_l;
    float scale_log2;                    // logit scale times log2(e)
    int residual;                        // fold dropped blocks (route present)
    const int32_t *kv_count, *kv_idx, *work_order;
    int n_items;                         // B * H * n_qb
    const uint32_t *kv_mask;
    const bf16 *kv_split;                // [BH][2][words][64][D] hi/lo residual tiles
    const float *k_bounds;               // [BH][words][2] key-mean and remainder norm bounds, or null (no early tests)
    float *lse;                          // nullable
    // fused routing (kv_idx unused): the decisions are taken in the kernel
    // from the block means and the pre-pass row statistics, and written out
    const float *q_mean, *k_mean, *row_stats;
    uint32_t *kv_mask_out;
    int32_t *kv_count_out;
    int tau_mode, n_prefix;
    int min_keep;                        // 0 or 1: the floor of one block
    float scale, ln_tau;
    int die_run_log2;                    // log2 of the work positions a die takes in a row (set at launch)
};

struct PermuteArgs {
    int N;                               // rows per (b, h)
    int units;                           // 16-byte units per row
    int n0, n_perm;                      // permuted rows [n0, n0 + n_perm)
    int inverse;                         // 0: gather, 1: scatter
};

hipError_t launch_pool(int dtype, int D, const void *q, const void *k, const void *v,
                       const PoolArgs &a, int BH, hipStream_t st);
// Proxy, selection and work order.  q == nullptr: centroid proxy (block means);
// otherwise the PAMA proxy from the queries q (dtype an sa_dtype).
hipError_t launch_select(int D, const SelectArgs &a, int BH, hipStream_t st, int dtype = 0,
                         const void *q = nullptr);
size_t pama_lds_bytes(int n_kb, int BQ, int dtype);
constexpr size_t kPamaLdsBudget = 128 * 1024;
constexpr int kFusedMaxWords = 512;              // decision words a fused work item holds in LDS
int select_group(int n_kb, int D, int n_qb);
size_t select_lds_bytes(int G, int n_kb, int D);
// Whether the route orders the work list head-major (else by cost band alone).
bool head_major_order(int BH, int n_qb);

// Sparse forward when a.kv_idx != nullptr, dense otherwise.
hipError_t launch_flash(int dtype, int D, int BQ, const void *q, const void *k, const void *v,
                        void *o, const FlashArgs &a, int BH, hipStream_t st);

// Probe-fitted residual correction.
constexpr int kPrMaxRank = 16;
constexpr int kPrChunk = 128;                    // probe rows per Gram workgroup
constexpr int kPrMaxPerBlock = 16;
struct PrArgs {
    int N, M, per_block, block_q, rank;  // M = n_qb * per_block probes per (b, h)
    float ridge;
    const float *O32;                    // [BH, N, D] sparse output (kept tokens only), fp32
    const float *Od32;                   // [BH, M, D] dense output at the probes, fp32
    float *scratch;                      // [BH, 3, D, D] Gram matrices
    int n_chunks;                        // probe chunks of kPrChunk rows per (b, h)
    float *part;                         // [BH, n_chunks, 3, D, D] Gram matrices of each chunk
    float *cmean;                        // [BH, n_chunks, 2, D] chunk means of x and r
    int kv_splits;                       // key ranges of the probe pass (1: written to Od32 directly)
    const float *Osplit;                 // [kv_splits, BH, M, D] probe outputs of each key range
    const float *Lsplit;                 // [kv_splits, BH, M] their log-sum-exp
    float *CB;                           // [BH, D, D] room: W = B Q [D][KP], then Q [D][KP]
    float *Cb;                           // [BH, D] b, then b Pk
};
// step 0: gather the probe queries of q into qp; 1: fit; 2: apply to o;
// 3: merge the probe pass's key ranges into Od32
hipError_t launch_sparsepr_step(int step, int dtype, int D, const void *q, void *qp, void *o, const PrArgs &a,
                                int BH, hipStream_t st);

// Token permutation on the GPU; host Hilbert order of a T x Hh x W grid on the
// 2^b cube (returns the number of points written to perm).
hipError_t launch_permute(const void *in, void *out, const int32_t *perm, const PermuteArgs &a, int BH,
                          hipStream_t st);
void hilbert_point(uint64_t h, int b, uint32_t X[3]);
int64_t hilbert_fill(int T, int Hh, int W, int b, int32_t *perm);

}  // namespace sa
