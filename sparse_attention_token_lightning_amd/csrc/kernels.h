// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
// Not installed; the public interface is include/ds4idx.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ds4idx {

enum { F32 = 0, BF16 = 1, FP8 = 2 };

struct Problem {
    int B, T, S, H, D;
    long long offset;  // query t sees keys s <= offset + t
    int q_dtype, k_dtype;
};

// Ragged batch: B streams packed along the rows of Q/W/idx (cu_q) and of K
// (cu_k); stream b's query t sees its keys s <= S_b - T_b + t.
struct VarlenProblem {
    int B, total_q;
    long long total_k;
    int max_k;  // >= every stream's S_b
    int H, D, q_dtype, k_dtype;
};

// Plain kernels: any H, D and dtype (the rollback path).
constexpr int kRefMaxQFloats = 16384;  // H*D + H floats of one query staged in LDS
hipError_t launch_score_ref(const Problem &p, const void *Q, const void *K, const float *Ks,
                            const float *W, float *scores, hipStream_t st);
hipError_t launch_topk_ref(const Problem &p, const float *scores, int k, int *idx, float *vals,
                           hipStream_t st);

// MFMA kernels: H = 64, D = 128, bf16 queries, bf16 or E4M3 keys.
constexpr int kMfmaH = 64, kMfmaD = 128, kMfmaMaxK = 512;
bool mfma_shape_ok(const Problem &p);
hipError_t launch_mfma_score(const Problem &p, const void *Q, const void *K, const float *Ks,
                             const float *W, float *scores, hipStream_t st);
hipError_t launch_mfma_select(const Problem &p, const void *Q, const void *K, const float *Ks,
                              const float *W, int k, int *idx, float *vals, hipStream_t st);
// fp8 x fp8 scorer: E4M3 queries with one fp32 scale per (token, head), E4M3 keys.
hipError_t launch_mfma_select_qfp8(const Problem &p, const void *Q8, const float *QS, const void *K, const float *Ks,
                                   const float *W, int k, int *idx, float *vals, hipStream_t st);
long long mfma_varlen_blocks(int B, int total_q);
// Ragged prefill with key parts: an 8-token block's visible keys are split
// into up to kPrefillMaxParts parts of kpart keys (a multiple of 128), each
// scored by its own workgroup, which publishes its exact top k per token; the
// last part to arrive merges. Workspace: [total_q] arrival counters (zero
// between calls), [total_q, kPrefillMaxParts] counts, [total_q,
// kPrefillMaxParts, k] (index << 32 | order key) entries.
constexpr int kPrefillMaxParts = 4;
struct PrefillParts {
    int kpart;  // keys per part; 0 = no parts
    uint64_t *list;
    uint32_t *cnt;
    uint32_t *ctr;
};
int set_prefill_split(int keys);  // -1 never, 0 automatic, > 0 part length; returns the previous value
int get_prefill_split();
int prefill_kpart(const VarlenProblem &p);  // 0: no parts for this problem
size_t prefill_parts_workspace_bytes(const VarlenProblem &p, int k);
hipError_t launch_mfma_select_varlen(const VarlenProblem &p, const int *cu_q, const long long *cu_k,
                                     const void *Q, const void *K, const float *Ks, const float *W,
                                     int k, int *idx, float *vals, void *ws, hipStream_t st);

// Split-key kernel for few rows over long caches (decode): partitions of
// 8192, 12288 or 16384 keys, each emitting a superset of its top k plus its
// m-th largest key; the last-arriving workgroup of a row merges.
constexpr int kSplitMaxParts = 256;
constexpr int kSplitPartLens[3] = {8192, 12288, 16384};
constexpr int kSplitCUs = 256;  // compute units of an MI355X: one split workgroup each
int set_split_len(int len);     // 0 = automatic; returns the previous value, -1 if unsupported
int get_split_len();
// Ragged batches of at most kSplitPlanRows query rows and streams, with the
// automatic length, take planned partitions: every row's keys split into
// equal parts of a length chosen on the device so that all parts start in
// one round on the kSplitCUs compute units (see the kernel).
constexpr int kSplitPlanRows = 256;
struct SplitWorkspace {
    uint32_t *ctr;         // [rows] arrival counters, zero between calls
    uint64_t *meta;        // [lists, 2] short-list edge << 32 | m-th largest key (~0: none); largest key
    uint64_t *full_list;   // [lists, slots] (index << 32 | order key), key 0 = empty slot
    uint64_t *short_list;  // [lists, short slots], same format
};                         // lists: rows x partitions per row, or the planned launch's blocks
// Rows of a split-key launch, the most keys a row sees, and the row length the
// merge's short lists are sized for (rows with fewer full partitions fall back
// to the full lists, which for short rows are few).
struct SplitShape {
    long long rows, max_len, short_len;
    int part;      // partition length (keys), one of kSplitPartLens; the longest for planned parts
    int plan = 0;  // planned parts: blocks launched (at least the parts of any plan), else 0
};
SplitShape split_shape(const Problem &p);
SplitShape split_shape(const VarlenProblem &p);
int split_slots(int k);
int split_short_slots(const SplitShape &sh, int k);
int split_parts(const SplitShape &sh);
size_t split_workspace_bytes(const SplitShape &sh, int k);
SplitWorkspace split_workspace(void *ws, const SplitShape &sh, int k);
hipError_t launch_split_select(const Problem &p, const void *Q, const void *K, const float *Ks,
                               const float *W, int k, int *idx, float *vals, void *ws, hipStream_t st);
hipError_t launch_split_select_varlen(const VarlenProblem &p, const int *cu_q, const long long *cu_k,
                                      const void *Q, const void *K, const float *Ks, const float *W, int k,
                                      int *idx, float *vals, void *ws, hipStream_t st);

// Allocation-free select: a fixed scratch array per GPU holds what the
// caller's workspace would (the split-key lists, or the plain path's scores).
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
void *noalloc_scratch();  // this device's scratch address (nullptr on failure)
hipError_t launch_zero_words(uint32_t *p, long long n, hipStream_t st);

// Sparse attention over selected positions of a shared latent cache: the key
// is the whole row (576 values), the value its first 512; heads in tiles of 64.
constexpr int kAttnHeadTile = 64, kAttnDqk = 576, kAttnDv = 512, kAttnMaxK = 2048;
struct AttnProblem {
    int B, T, S, H, topk;
    float softmax_scale;
};
hipError_t launch_sparse_attention(const AttnProblem &p, const void *Q, const void *KV, const int *idx, void *O,
                                   float *lse, hipStream_t st);

// Key-cache writer: per-token E4M3 quantisation, V values on each of G lanes per token.
int k_cache_lanes(int D, int V);
int k_cache_vals_per_lane(int D, const void *cache);
hipError_t launch_k_cache_write(const void *kin, int k_dtype, long long n, int D,
                                const long long *slots, uint8_t *cache, float *cache_scale,
                                long long rows, hipStream_t st);

}  // namespace ds4idx
