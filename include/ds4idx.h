/*
 * ds4idx — the Lightning Indexer of DeepSeek V4's sparse attention, as a C-ABI
 * library of hand-written HIP kernels for AMD MI355X (gfx950).
 *
 * What it computes. For every query token the indexer scores all causally
 * visible cached keys and keeps the positions worth attending to; the pages
 * describe it as the step that dominates long-context prefill, made of a
 * scorer and a top-512 selection (first page, "DeepSeek V4 Flash 추론을 1.6초로
 * 줄인 ds4 최적화": glossary entry "Lightning Indexer"; section details, second
 * paragraph). The score is the indexer's published form
 *
 *     score(t, s) = sum_h W[t,h] * max(0, sum_d Q[t,h,d] * K[s,d] * K_scale[s])
 *
 * and query t of a call, whose absolute position is causal_offset + t, sees the
 * keys s <= causal_offset + t. The selection keeps the min(k, L) visible keys
 * (L = causal_offset + t + 1) that come first in the strict order (score
 * descending, index ascending): equal scores go to the lower index. Because the
 * order is total, the answer is unique, as the pages' byte-identical outputs
 * across kernel rewrites require (first page, TL;DR).
 *
 * Layouts (row-major, contiguous, device memory owned by the caller):
 *   Q        [B, T, H, D]  fp32 or bf16                       16-byte aligned
 *   K        [B, S, D]     fp32, bf16, or OCP E4M3FN codes    16-byte aligned
 *   K_scale  [B, S]        fp32, positive finite; required for E4M3 keys
 *                          (ignored, may be NULL, otherwise)
 *   W        [B, T, H]     fp32 head weights
 *   scores   [B, T, S]     fp32 (ds4idx_score output; -inf where s is masked)
 *   idx      [B, T, k]     int32: selected key indices in ascending order,
 *                          then -1 padding after min(k, L) entries
 *   vals     [B, T, k]     fp32 scores of idx (-inf in padding); may be NULL
 *
 * FP8 keys are OCP E4M3FN (bias 7, max 448, NaN = S.1111.111, no infinities),
 * never the FNUZ variant: the MI300X write-up ("DeepSeek V4 Flash는 단일 AMD
 * MI300X에서 실행됩니다", section on the indexer cache's FP8 format mismatch)
 * shows that mixing the two readings scales every key by 2.
 *
 * Calls are asynchronous on the HIP stream passed as `stream` (a hipStream_t;
 * NULL = the default stream). The return value reports argument validation
 * and launch errors only; device faults surface at the caller's next
 * synchronisation. Every argument is validated before any HIP call is made.
 * The library never allocates, frees or synchronises in these calls, keeps no
 * pointer after returning, and is safe to call from several threads on
 * different streams. Non-finite Q, K or W values give undefined (but
 * memory-safe) results.
 */
#ifndef DS4IDX_H
#define DS4IDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DS4IDX_ABI_VERSION 1
#define DS4IDX_MAX_TOPK 2048
#define DS4IDX_K_CACHE_MAX_D 512 /* largest D ds4idx_k_cache_write takes */

typedef enum {
    DS4IDX_OK = 0,
    DS4IDX_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad k */
    DS4IDX_ERR_UNSUPPORTED = 2, /* shape/dtype with no kernel under the forced implementation */
    DS4IDX_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than ds4idx_workspace_bytes */
    DS4IDX_ERR_HIP = 4,         /* a HIP launch or query failed */
    DS4IDX_ERR_SCRATCH = 5      /* ds4idx_select_noalloc: needs more than DS4IDX_NOALLOC_SCRATCH_BYTES */
} ds4idx_status;

typedef enum {
    DS4IDX_F32 = 0,
    DS4IDX_BF16 = 1,
    DS4IDX_FP8_E4M3 = 2 /* OCP E4M3FN codes, one byte each; keys only */
} ds4idx_dtype;

/* Problem shape shared by every entry point. All sizes >= 1, causal_offset
 * >= 0 and causal_offset + T <= S (the cache already holds the new tokens).
 * Key indices are int32, so S <= 2^31 - 1; internal offsets are 64-bit. */
typedef struct {
    int32_t B, T, S, H, D;
    int64_t causal_offset;
    int32_t q_dtype; /* ds4idx_dtype: F32 or BF16 */
    int32_t k_dtype; /* ds4idx_dtype: F32, BF16 or FP8_E4M3 */
} ds4idx_problem;

enum { DS4IDX_OP_SCORE = 0, DS4IDX_OP_TOPK = 1, DS4IDX_OP_SELECT = 2 };

/* Kernel family. AUTO: the MFMA kernels where the shape allows, the plain
 * kernels otherwise. REF: the plain kernels for every shape. OPT: the MFMA
 * kernels only; shapes they do not cover return DS4IDX_ERR_UNSUPPORTED.
 * The pages keep each new kernel behind a rollback switch so the old path
 * stays comparable (first page, practical advice, third paragraph); this is
 * that switch. Its initial value comes from the environment variable
 * DS4IDX_IMPL ("auto", "ref" or "opt"; default "auto"). */
enum { DS4IDX_IMPL_AUTO = 0, DS4IDX_IMPL_REF = 1, DS4IDX_IMPL_OPT = 2 };

/* ABI version of the loaded library (DS4IDX_ABI_VERSION). */
int ds4idx_abi_version(void);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char *ds4idx_status_string(int status);

/* Select the kernel family for later calls in this process; returns the
 * previous value, or -1 for an unknown value (then nothing changes). */
int ds4idx_set_impl(int impl);
int ds4idx_get_impl(void);

/* Partition length of the split-key kernel, the kernel for problems with few
 * query rows over long caches (decode): each workgroup scores one partition
 * of a row's keys and the last one to finish merges the row. Lengths 8192,
 * 12288 and 16384 keys are built; 0 (the default) lets the library pick per
 * call the shortest length whose partitions all start in one round on the
 * GPU's compute units (one partition per unit), using for ragged batches with
 * one query per stream the bound total_k / length + B. A fixed length is for
 * measurement and comparison: results are identical for every length. The
 * workspace size depends on the length, so query ds4idx_workspace_bytes (or
 * ds4idx_varlen_workspace_bytes) after changing it. The initial value comes
 * from the environment variable DS4IDX_SPLIT (a length in keys; anything
 * else means automatic). ds4idx_set_split returns the previous value, or -1
 * for an unsupported length (then nothing changes). */
int ds4idx_set_split(int keys);
int ds4idx_get_split(void);

/* Key parts for ragged prefill batches (ds4idx_select_varlen on the prefill
 * kernel): in a small batch the 8-token blocks of the longest caches set the
 * pace while other compute units idle, so each block's visible keys can be
 * split into up to 4 parts, each scored by its own workgroup; the part that
 * finishes last merges the parts' exact selections per token (the result is
 * identical to the unsplit one). 0 (default): parts of 8192 keys when the
 * longest cache exceeds 8192 keys and the batch has at most two rounds of
 * blocks for the GPU's compute units; -1: never; a positive value: parts of
 * that many keys (rounded up to a multiple of 128, and at least a quarter of
 * max_k). Parts need workspace, so query ds4idx_varlen_workspace_bytes after
 * changing this. Initial value from the environment variable
 * DS4IDX_PREFILL_SPLIT. ds4idx_set_prefill_split returns the previous value. */
int ds4idx_set_prefill_split(int keys);
int ds4idx_get_prefill_split(void);

/* Bytes of device workspace that `op` (DS4IDX_OP_*) needs for this problem
 * and k under the current kernel family, or 0 if it needs none. Returns
 * (size_t)-1 for an invalid problem. The workspace for DS4IDX_OP_SELECT must
 * be zero-filled before its first use (it holds per-row arrival counters that
 * every completed call leaves at zero again); 256-byte alignment required. */
size_t ds4idx_workspace_bytes(const ds4idx_problem *p, int32_t k, int32_t op);

/* Scorer only: scores[b,t,s] for every s in [0, S): the score of visible keys
 * (s <= causal_offset + t) and -inf for the rest. */
int ds4idx_score(const ds4idx_problem *p, const void *Q, const void *K, const float *K_scale,
                 const float *W, float *scores, void *stream);

/* Top-k over materialised scores [B,T,S] (only the visible prefix of each row,
 * s <= causal_offset + t, is read). 1 <= k <= DS4IDX_MAX_TOPK. Uses no
 * workspace (workspace may be NULL). */
int ds4idx_topk(const ds4idx_problem *p, const float *scores, int32_t k, int32_t *idx,
                float *vals, void *workspace, size_t ws_bytes, void *stream);

/* Fused scorer + top-k: the indexer's hot path. Same outputs as
 * ds4idx_score followed by ds4idx_topk, without materialising the scores
 * when the MFMA kernels apply (H = 64, D = 128, bf16 Q, bf16 or E4M3 K,
 * k <= 512). 1 <= k <= DS4IDX_MAX_TOPK. */
int ds4idx_select(const ds4idx_problem *p, const void *Q, const void *K, const float *K_scale,
                  const float *W, int32_t k, int32_t *idx, float *vals, void *workspace,
                  size_t ws_bytes, void *stream);

/* Allocation-free fused select, for callers that cannot allocate device
 * memory around the call: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, outputs and kernels as
 * ds4idx_select, without the workspace: the workspace the call would need
 * (the split-key kernel's per-row counters and candidate lists, or the plain
 * kernels' score matrix) lives in a fixed array of
 * DS4IDX_NOALLOC_SCRATCH_BYTES in device memory that the library holds on
 * each GPU it runs on until the process ends. The call allocates nothing and
 * frees nothing; it clears the words that must start at zero with a fill
 * kernel on `stream` before the selection kernel.
 *
 * Problems whose workspace (ds4idx_workspace_bytes) exceeds the array return
 * DS4IDX_ERR_SCRATCH before any HIP call; the prefill kernel's problems need
 * none. The array belongs to the device current on the calling thread, which
 * must be the device of `stream`. Every call on a GPU shares that GPU's
 * array: calls whose executions overlap on one GPU (other streams, other
 * threads) race and give undefined results; calls in one stream are
 * ordered. */
#define DS4IDX_NOALLOC_SCRATCH_BYTES (32u << 20)
int ds4idx_select_noalloc(const ds4idx_problem *p, const void *Q, const void *K, const float *K_scale,
                          const float *W, int32_t k, int32_t *idx, float *vals, void *stream);

/* Ragged batch: B independent streams (requests) packed along the rows, in
 * one launch, as a serving step mixes requests with different cache lengths
 * and different numbers of new tokens (the MI300X write-up's concurrency
 * sweep and chunked-prefill token budget, "DeepSeek V4 Flash는 단일 AMD
 * MI300X에서 실행됩니다", production tuning table). Stream b owns query rows
 * cu_q[b] .. cu_q[b+1]-1 of Q, W, idx and vals (T_b rows) and key rows
 * cu_k[b] .. cu_k[b+1]-1 of K and K_scale (S_b cached keys). Its new tokens
 * are the last T_b of its cache, so its query t sees its keys
 * s <= S_b - T_b + t, and idx holds indices local to the stream (0 .. S_b-1),
 * ascending, -1 padded, as in ds4idx_select. Each stream's result equals a
 * ds4idx_select call on that stream alone with causal_offset = S_b - T_b.
 *
 * Layouts: Q [total_q, H, D], W [total_q, H], K [total_k, D], K_scale
 * [total_k], idx and vals [total_q, k]. cu_q (int32) and cu_k (int64) are
 * device arrays of B + 1 non-decreasing prefix sums from 0 to total_q and
 * total_k; T_b <= S_b <= max_k is required. Malformed prefix arrays give
 * undefined results for the rows concerned, but no access outside the
 * buffers the sizes describe. Only the MFMA shape has ragged kernels (H = 64,
 * D = 128, bf16 Q, bf16 or E4M3 K); other shapes return
 * DS4IDX_ERR_UNSUPPORTED, and the kernel-family switch does not apply. */
typedef struct {
    int32_t B;           /* streams, >= 1 */
    int32_t total_q;     /* cu_q[B]: query rows (0: nothing to do) */
    int64_t total_k;     /* cu_k[B]: key rows */
    int32_t max_k;       /* >= every S_b: sizes the split-key grid and workspace */
    int32_t H, D;
    int32_t q_dtype, k_dtype;
} ds4idx_varlen_problem;

/* Workspace bytes for ds4idx_select_varlen (0 if none), or (size_t)-1 for an
 * invalid problem: the split-key kernel's lists, or the prefill kernel's key
 * parts (see ds4idx_set_prefill_split). Same zero-fill and alignment rules as
 * ds4idx_select's. */
size_t ds4idx_varlen_workspace_bytes(const ds4idx_varlen_problem *p, int32_t k);

/* Fused scorer + top-k over a ragged batch (see above). 1 <= k <= DS4IDX_MAX_TOPK;
 * k > 512 is served only when the batch has few enough rows for the split-key
 * kernel (total_q <= 65535). */
int ds4idx_select_varlen(const ds4idx_varlen_problem *p, const int32_t *cu_q, const int64_t *cu_k,
                         const void *Q, const void *K, const float *K_scale, const float *W,
                         int32_t k, int32_t *idx, float *vals, void *workspace, size_t ws_bytes,
                         void *stream);

/* fp8 x fp8 scorer + top-k: ds4idx_select with the queries, too, in OCP
 * E4M3, one fp32 scale per (token, head), and the E4M3 matrix-core path
 * (twice the bf16 peak on gfx950). The score is computed from the dequantised
 * queries Q_scale[b,t,h] * decode(Q8[b,t,h,d]); rounding Q to a 3-bit
 * mantissa moves scores by about 2%, so the selection is close to, not equal
 * to, the bf16-query selection (the survey's fp8 x fp8 variant; the parity
 * cost is measured and reported beside the benchmark). Quantise the queries
 * with ds4idx_k_cache_write over their B*T*H rows of D values.
 *   Q8       [B, T, H, D] E4M3 codes, 16-byte aligned
 *   Q_scale  [B, T, H]    fp32, positive finite
 * Other arguments as for ds4idx_select; p->q_dtype and p->k_dtype must both be
 * DS4IDX_FP8_E4M3. Kernel shape: H = 64, D = 128, k <= 512 (otherwise
 * DS4IDX_ERR_UNSUPPORTED); no workspace. */
int ds4idx_select_qfp8(const ds4idx_problem *p, const void *Q8, const float *Q_scale, const void *K,
                       const float *K_scale, const float *W, int32_t k, int32_t *idx, float *vals,
                       void *stream);

/* Sparse attention over the selected positions, the step downstream of the
 * indexer: each query token attends only to the cache rows its idx row names
 * (first page, glossary entry on sparse attention). The MI300X write-up keeps
 * an MLA cache (fp8_ds_mla) and tiles the sparse prefill 64 heads at a time
 * (BLOCK_H=64 in its production tuning table); it prints no formula. Here
 * each cache row is one shared latent vector: the whole row (d_qk values) is
 * the key of every head and its first d_v values the value:
 *
 *     z_j        = softmax_scale * sum_d Q[b,t,h,d] * KV[b, idx_j, d]
 *     O[b,t,h,:] = sum_j exp(z_j) KV[b, idx_j, 0:d_v] / sum_j exp(z_j)
 *     lse[b,t,h] = log(sum_j exp(z_j))           (natural log)
 *
 * over the entries j of idx[b,t,:] with 0 <= idx < S; -1 padding (as
 * ds4idx_select emits) and other out-of-range entries are skipped, and a
 * token with none gets O = 0 and lse = -inf.
 *   Q    [B, T, H, d_qk] bf16, 16-byte aligned
 *   KV   [B, S, d_qk]    bf16, 16-byte aligned
 *   idx  [B, T, topk]    int32 (e.g. ds4idx_select's output)
 *   O    [B, T, H, d_v]  bf16, 16-byte aligned
 *   lse  [B, T, H]       fp32, may be NULL
 * Probabilities enter the value sum rounded to bf16 (accumulation in fp32).
 * The kernel covers d_qk = 576, d_v = 512 (a 512-value latent plus a
 * 64-value positional part) and H a multiple of 64; other shapes return
 * DS4IDX_ERR_UNSUPPORTED. 1 <= topk <= DS4IDX_MAX_TOPK. */
typedef struct {
    int32_t B, T, S, H, topk;
    int32_t d_qk, d_v;
    float softmax_scale;
} ds4idx_attn_problem;

int ds4idx_sparse_attention(const ds4idx_attn_problem *p, const void *Q, const void *KV,
                            const int32_t *idx, void *O, float *lse, void *stream);

/* Key-cache writer, the step upstream of the scorer: quantises n new key
 * vectors to OCP E4M3FN codes with one fp32 scale per token and stores them in
 * rows of the key cache that ds4idx_select reads as K and K_scale. The pages
 * record that the indexer's cache holds E4M3 codes and that reading codes of
 * one E4M3 variant as the other scales every key by 2 (MI300X write-up, FP8
 * format mismatch section); they do not print a scale rule. The rule here is
 * plain absmax scaling into the OCP range:
 *
 *     scale[s]  = max(amax_s, 2^-126) / 448      amax_s = max_d |K_new[s,d]|
 *     code[s,d] = E4M3 round-to-nearest-even of clamp(K_new[s,d] / scale[s], -448, 448)
 *
 * both divisions in correctly rounded fp32; a zero result keeps its sign
 * (-0 gives 0x80). Dequantised keys are scale[s] * decode(code[s,d]).
 *
 *   K_new        [n, D] fp32 or bf16 (k_dtype DS4IDX_F32 or DS4IDX_BF16),
 *                16-byte aligned
 *   slots        [n] int64 device array: the cache row each token goes to, or
 *                NULL for rows 0 .. n-1. Tokens whose slot lies outside
 *                [0, cache_rows) are skipped (nothing written); two tokens
 *                with the same slot race.
 *   cache        [cache_rows, D] E4M3 codes, 8-byte aligned
 *   cache_scale  [cache_rows] fp32
 *
 * D must be a multiple of 8 and at most 512, n >= 0 (n = 0 launches nothing),
 * cache_rows >= 1. Non-finite inputs give undefined codes. Asynchronous on
 * `stream`, like the other calls; no workspace. */
int ds4idx_k_cache_write(const void *K_new, int32_t k_dtype, int64_t n, int32_t D,
                         const int64_t *slots, uint8_t *cache, float *cache_scale,
                         int64_t cache_rows, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DS4IDX_H */
