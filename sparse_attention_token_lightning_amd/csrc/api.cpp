// C-ABI entry points of libds4idx (declared in include/ds4idx.h): argument
// validation (always before any HIP call), workspace sizing, and dispatch to
// the MFMA kernels or the plain kernels.
#include "ds4idx.h"

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "kernels.h"

using ds4idx::Problem;

static_assert(DS4IDX_NOALLOC_SCRATCH_BYTES == ds4idx::kNoallocScratchBytes,
              "the header states the scratch array's size");

namespace {

std::atomic<int> g_impl{-1};

int impl_now()
{
    int v = g_impl.load(std::memory_order_relaxed);
    if (v >= 0) return v;
    int init = DS4IDX_IMPL_AUTO;
    if (const char *e = std::getenv("DS4IDX_IMPL")) {
        if (!std::strcmp(e, "ref")) init = DS4IDX_IMPL_REF;
        else if (!std::strcmp(e, "opt")) init = DS4IDX_IMPL_OPT;
    }
    int expected = -1;
    g_impl.compare_exchange_strong(expected, init);
    return g_impl.load(std::memory_order_relaxed);
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_problem(const ds4idx_problem *p)
{
    if (!p) return DS4IDX_ERR_INVALID_ARG;
    if (p->B < 1 || p->T < 1 || p->S < 1 || p->H < 1 || p->D < 1) return DS4IDX_ERR_INVALID_ARG;
    if (p->causal_offset < 0 || p->causal_offset + (int64_t)p->T > (int64_t)p->S)
        return DS4IDX_ERR_INVALID_ARG;
    if (p->q_dtype != DS4IDX_F32 && p->q_dtype != DS4IDX_BF16) return DS4IDX_ERR_INVALID_ARG;
    if (p->k_dtype != DS4IDX_F32 && p->k_dtype != DS4IDX_BF16 && p->k_dtype != DS4IDX_FP8_E4M3)
        return DS4IDX_ERR_INVALID_ARG;
    // The grid's x dimension carries B*T rows (top-k) or B*T*key-blocks (scorer).
    if ((int64_t)p->B * p->T > (int64_t)INT32_MAX) return DS4IDX_ERR_UNSUPPORTED;
    return DS4IDX_OK;
}

int check_inputs(const ds4idx_problem *p, const void *Q, const void *K, const float *Ks,
                 const float *W)
{
    if (!Q || !K || !W) return DS4IDX_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(W, 4)) return DS4IDX_ERR_INVALID_ARG;
    if (p->k_dtype == DS4IDX_FP8_E4M3 && (!Ks || !aligned(Ks, 4))) return DS4IDX_ERR_INVALID_ARG;
    return DS4IDX_OK;
}

Problem to_internal(const ds4idx_problem *p)
{
    return Problem{p->B, p->T, p->S, p->H, p->D, (long long)p->causal_offset, p->q_dtype, p->k_dtype};
}

bool ref_shape_ok(const ds4idx_problem *p)
{
    if ((int64_t)p->H * p->D + p->H > ds4idx::kRefMaxQFloats) return false;
    const int64_t key_blocks = ((int64_t)p->S + 1023) / 1024;
    return (int64_t)p->B * p->T * key_blocks <= (int64_t)INT32_MAX;
}

// Which kernels a call takes: 1 = MFMA, 0 = plain, -1 = none under the forced family.
int route_score(const ds4idx_problem *p)
{
    const Problem q = to_internal(p);
    const int impl = impl_now();
    const bool mf = ds4idx::mfma_shape_ok(q);
    if (impl == DS4IDX_IMPL_OPT) return mf ? 1 : -1;
    if (impl == DS4IDX_IMPL_AUTO && mf) return 1;
    return ref_shape_ok(p) ? 0 : -1;
}

enum Route { R_NONE = -1, R_REF = 0, R_PREFILL = 1, R_SPLIT = 2 };

// Fused select: the MFMA prefill kernel (8 query tokens per workgroup, whole
// rows) when there are enough rows to fill the GPU; the split-key kernel when
// there are too few rows (decode); the plain kernels otherwise.
int route_select(const ds4idx_problem *p, int32_t k)
{
    const Problem q = to_internal(p);
    const int impl = impl_now();
    const bool shape = ds4idx::mfma_shape_ok(q);
    const int64_t rows = (int64_t)p->B * p->T;
    const bool prefill_ok = shape && k <= ds4idx::kMfmaMaxK && p->B <= 65535;
    const bool split_ok =
        shape && rows <= 65535 && ds4idx::split_parts(ds4idx::split_shape(q)) <= ds4idx::kSplitMaxParts;
    const int64_t prefill_blocks = (int64_t)p->B * ((p->T + 7) / 8);
    int mf = R_NONE;
    if (split_ok && (prefill_blocks < 128 || !prefill_ok)) mf = R_SPLIT;
    else if (prefill_ok) mf = R_PREFILL;
    if (impl == DS4IDX_IMPL_OPT) return mf;
    if (impl == DS4IDX_IMPL_AUTO && mf != R_NONE) return mf;
    return ref_shape_ok(p) ? R_REF : R_NONE;
}

size_t round_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

// Plain select path: materialised scores [B,T,S] fp32.
size_t ref_select_bytes(const ds4idx_problem *p)
{
    return round_up((size_t)p->B * p->T * p->S * sizeof(float), 256);
}

int launch_status(hipError_t e) { return e == hipSuccess ? DS4IDX_OK : DS4IDX_ERR_HIP; }

int check_varlen(const ds4idx_varlen_problem *p)
{
    if (!p) return DS4IDX_ERR_INVALID_ARG;
    if (p->B < 1 || p->total_q < 0 || p->total_k < 0 || p->max_k < 1 || p->H < 1 || p->D < 1)
        return DS4IDX_ERR_INVALID_ARG;
    if (p->q_dtype != DS4IDX_F32 && p->q_dtype != DS4IDX_BF16) return DS4IDX_ERR_INVALID_ARG;
    if (p->k_dtype != DS4IDX_F32 && p->k_dtype != DS4IDX_BF16 && p->k_dtype != DS4IDX_FP8_E4M3)
        return DS4IDX_ERR_INVALID_ARG;
    return DS4IDX_OK;
}

ds4idx::VarlenProblem to_internal(const ds4idx_varlen_problem *p)
{
    return ds4idx::VarlenProblem{p->B, p->total_q, (long long)p->total_k, p->max_k, p->H, p->D,
                                 p->q_dtype, p->k_dtype};
}

// Ragged select: the split-key kernel for few rows (decode batches), the
// prefill kernel otherwise; only the MFMA shape has ragged kernels.
int route_varlen(const ds4idx_varlen_problem *p, int32_t k)
{
    const ds4idx::VarlenProblem v = to_internal(p);
    const bool shape = v.H == ds4idx::kMfmaH && v.D == ds4idx::kMfmaD && v.q_dtype == DS4IDX_BF16 &&
                       (v.k_dtype == DS4IDX_BF16 || v.k_dtype == DS4IDX_FP8_E4M3);
    if (!shape) return R_NONE;
    const long long blocks = ds4idx::mfma_varlen_blocks(v.B, v.total_q);
    const bool prefill_ok = k <= ds4idx::kMfmaMaxK && blocks * ds4idx::kPrefillMaxParts <= (long long)INT32_MAX;
    const bool split_ok = v.total_q <= 65535 &&
                          ds4idx::split_parts(ds4idx::split_shape(v)) <= ds4idx::kSplitMaxParts;
    if (split_ok && (blocks < 128 || !prefill_ok)) return R_SPLIT;
    return prefill_ok ? R_PREFILL : R_NONE;
}

}  // namespace

extern "C" {

int ds4idx_abi_version(void) { return DS4IDX_ABI_VERSION; }

const char *ds4idx_status_string(int status)
{
    switch (status) {
    case DS4IDX_OK: return "ok";
    case DS4IDX_ERR_INVALID_ARG: return "invalid argument";
    case DS4IDX_ERR_UNSUPPORTED: return "unsupported shape or dtype for the selected kernels";
    case DS4IDX_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case DS4IDX_ERR_HIP: return "HIP launch or runtime error";
    case DS4IDX_ERR_SCRATCH:
        return "problem needs more scratch memory than the allocation-free entry point holds";
    default: return "unknown status";
    }
}

int ds4idx_set_impl(int impl)
{
    if (impl != DS4IDX_IMPL_AUTO && impl != DS4IDX_IMPL_REF && impl != DS4IDX_IMPL_OPT) return -1;
    const int prev = impl_now();
    g_impl.store(impl, std::memory_order_relaxed);
    return prev;
}

int ds4idx_get_impl(void) { return impl_now(); }

int ds4idx_set_split(int keys) { return ds4idx::set_split_len(keys); }

int ds4idx_get_split(void) { return ds4idx::get_split_len(); }

int ds4idx_set_prefill_split(int keys) { return ds4idx::set_prefill_split(keys); }

int ds4idx_get_prefill_split(void) { return ds4idx::get_prefill_split(); }

size_t ds4idx_workspace_bytes(const ds4idx_problem *p, int32_t k, int32_t op)
{
    if (check_problem(p) != DS4IDX_OK) return (size_t)-1;
    if (op == DS4IDX_OP_SCORE || op == DS4IDX_OP_TOPK) return 0;
    if (op != DS4IDX_OP_SELECT || k < 1 || k > DS4IDX_MAX_TOPK) return (size_t)-1;
    const int r = route_select(p, k);
    if (r == R_REF) return ref_select_bytes(p);
    if (r == R_SPLIT) return ds4idx::split_workspace_bytes(ds4idx::split_shape(to_internal(p)), k);
    return 0;
}

int ds4idx_score(const ds4idx_problem *p, const void *Q, const void *K, const float *K_scale,
                 const float *W, float *scores, void *stream)
{
    int st = check_problem(p);
    if (st != DS4IDX_OK) return st;
    if ((st = check_inputs(p, Q, K, K_scale, W)) != DS4IDX_OK) return st;
    if (!scores || !aligned(scores, 4)) return DS4IDX_ERR_INVALID_ARG;
    const int r = route_score(p);
    if (r < 0) return DS4IDX_ERR_UNSUPPORTED;
    const Problem q = to_internal(p);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (r == 1) return launch_status(ds4idx::launch_mfma_score(q, Q, K, K_scale, W, scores, s));
    return launch_status(ds4idx::launch_score_ref(q, Q, K, K_scale, W, scores, s));
}

int ds4idx_topk(const ds4idx_problem *p, const float *scores, int32_t k, int32_t *idx, float *vals,
                void *workspace, size_t ws_bytes, void *stream)
{
    (void)workspace;
    (void)ws_bytes;
    int st = check_problem(p);
    if (st != DS4IDX_OK) return st;
    if (k < 1 || k > DS4IDX_MAX_TOPK) return DS4IDX_ERR_INVALID_ARG;
    if (!scores || !idx || !aligned(scores, 4) || !aligned(idx, 4) || (vals && !aligned(vals, 4)))
        return DS4IDX_ERR_INVALID_ARG;
    const Problem q = to_internal(p);
    return launch_status(ds4idx::launch_topk_ref(q, scores, k, idx, vals, static_cast<hipStream_t>(stream)));
}

int ds4idx_select(const ds4idx_problem *p, const void *Q, const void *K, const float *K_scale,
                  const float *W, int32_t k, int32_t *idx, float *vals, void *workspace,
                  size_t ws_bytes, void *stream)
{
    int st = check_problem(p);
    if (st != DS4IDX_OK) return st;
    if ((st = check_inputs(p, Q, K, K_scale, W)) != DS4IDX_OK) return st;
    if (k < 1 || k > DS4IDX_MAX_TOPK) return DS4IDX_ERR_INVALID_ARG;
    if (!idx || !aligned(idx, 4) || (vals && !aligned(vals, 4))) return DS4IDX_ERR_INVALID_ARG;
    const int r = route_select(p, k);
    if (r == R_NONE) return DS4IDX_ERR_UNSUPPORTED;
    const Problem q = to_internal(p);
    const size_t need = r == R_REF ? ref_select_bytes(p)
                        : r == R_SPLIT ? ds4idx::split_workspace_bytes(ds4idx::split_shape(q), k) : 0;
    if (need > 0 && (!workspace || !aligned(workspace, 256) || ws_bytes < need))
        return DS4IDX_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (r == R_PREFILL)
        return launch_status(ds4idx::launch_mfma_select(q, Q, K, K_scale, W, k, idx, vals, s));
    if (r == R_SPLIT)
        return launch_status(ds4idx::launch_split_select(q, Q, K, K_scale, W, k, idx, vals, workspace, s));
    float *sc = static_cast<float *>(workspace);
    st = launch_status(ds4idx::launch_score_ref(q, Q, K, K_scale, W, sc, s));
    if (st != DS4IDX_OK) return st;
    return launch_status(ds4idx::launch_topk_ref(q, sc, k, idx, vals, s));
}

int ds4idx_select_noalloc(const ds4idx_problem *p, const void *Q, const void *K, const float *K_scale,
                          const float *W, int32_t k, int32_t *idx, float *vals, void *stream)
{
    int st = check_problem(p);
    if (st != DS4IDX_OK) return st;
    if ((st = check_inputs(p, Q, K, K_scale, W)) != DS4IDX_OK) return st;
    if (k < 1 || k > DS4IDX_MAX_TOPK) return DS4IDX_ERR_INVALID_ARG;
    if (!idx || !aligned(idx, 4) || (vals && !aligned(vals, 4))) return DS4IDX_ERR_INVALID_ARG;
    const int r = route_select(p, k);
    if (r == R_NONE) return DS4IDX_ERR_UNSUPPORTED;
    const Problem q = to_internal(p);
    const size_t need = r == R_REF ? ref_select_bytes(p)
                        : r == R_SPLIT ? ds4idx::split_workspace_bytes(ds4idx::split_shape(q), k) : 0;
    if (need > ds4idx::kNoallocScratchBytes) return DS4IDX_ERR_SCRATCH;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (r == R_PREFILL)
        return launch_status(ds4idx::launch_mfma_select(q, Q, K, K_scale, W, k, idx, vals, s));
    void *ws = ds4idx::noalloc_scratch();
    if (!ws) return DS4IDX_ERR_HIP;
    if (r == R_SPLIT) {
        // Only the arrival counters must start at zero; every other word of
        // the split-key workspace is written before it is read.
        const ds4idx::SplitShape sh = ds4idx::split_shape(q);
        st = launch_status(
            ds4idx::launch_zero_words(ds4idx::split_workspace(ws, sh, k).ctr, sh.rows, s));
        if (st != DS4IDX_OK) return st;
        return launch_status(ds4idx::launch_split_select(q, Q, K, K_scale, W, k, idx, vals, ws, s));
    }
    float *sc = static_cast<float *>(ws);
    st = launch_status(ds4idx::launch_score_ref(q, Q, K, K_scale, W, sc, s));
    if (st != DS4IDX_OK) return st;
    return launch_status(ds4idx::launch_topk_ref(q, sc, k, idx, vals, s));
}

int ds4idx_k_cache_write(const void *K_new, int32_t k_dtype, int64_t n, int32_t D,
                         const int64_t *slots, uint8_t *cache, float *cache_scale,
                         int64_t cache_rows, void *stream)
{
    if (k_dtype != DS4IDX_F32 && k_dtype != DS4IDX_BF16) return DS4IDX_ERR_INVALID_ARG;
    if (n < 0 || D < 8 || D % 8 != 0 || D > DS4IDX_K_CACHE_MAX_D || cache_rows < 1)
        return DS4IDX_ERR_INVALID_ARG;
    if (n == 0) return DS4IDX_OK;
    if (!K_new || !cache || !cache_scale || !aligned(K_new, 16) || !aligned(cache, 8) ||
        !aligned(cache_scale, 4) || (slots && !aligned(slots, 8)))
        return DS4IDX_ERR_INVALID_ARG;
    // One 256-thread block per 256 / G tokens; the grid's x dimension is 32-bit.
    const int G = ds4idx::k_cache_lanes(D, ds4idx::k_cache_vals_per_lane(D, cache));
    if (n > ((int64_t)INT32_MAX / G) * 256) return DS4IDX_ERR_UNSUPPORTED;
    static_assert(sizeof(long long) == sizeof(int64_t), "int64 slots");
    return launch_status(ds4idx::launch_k_cache_write(K_new, k_dtype, n, D,
                                                      reinterpret_cast<const long long *>(slots),
                                                      cache, cache_scale, cache_rows,
                                                      static_cast<hipStream_t>(stream)));
}

size_t ds4idx_varlen_workspace_bytes(const ds4idx_varlen_problem *p, int32_t k)
{
    if (check_varlen(p) != DS4IDX_OK || k < 1 || k > DS4IDX_MAX_TOPK) return (size_t)-1;
    if (p->total_q == 0) return 0;
    const int r = route_varlen(p, k);
    if (r == R_PREFILL) return ds4idx::prefill_parts_workspace_bytes(to_internal(p), k);
    if (r != R_SPLIT) return 0;
    return ds4idx::split_workspace_bytes(ds4idx::split_shape(to_internal(p)), k);
}

int ds4idx_select_varlen(const ds4idx_varlen_problem *p, const int32_t *cu_q, const int64_t *cu_k,
                         const void *Q, const void *K, const float *K_scale, const float *W, int32_t k,
                         int32_t *idx, float *vals, void *workspace, size_t ws_bytes, void *stream)
{
    int st = check_varlen(p);
    if (st != DS4IDX_OK) return st;
    if (k < 1 || k > DS4IDX_MAX_TOPK) return DS4IDX_ERR_INVALID_ARG;
    if (!cu_q || !cu_k || !aligned(cu_q, 4) || !aligned(cu_k, 8)) return DS4IDX_ERR_INVALID_ARG;
    if (!Q || !K || !W || !idx || !aligned(Q, 16) || !aligned(K, 16) || !aligned(W, 4) || !aligned(idx, 4) ||
        (vals && !aligned(vals, 4)))
        return DS4IDX_ERR_INVALID_ARG;
    if (p->k_dtype == DS4IDX_FP8_E4M3 && (!K_scale || !aligned(K_scale, 4))) return DS4IDX_ERR_INVALID_ARG;
    const int r = route_varlen(p, k);
    if (r == R_NONE) return DS4IDX_ERR_UNSUPPORTED;
    if (p->total_q == 0) return DS4IDX_OK;
    const ds4idx::VarlenProblem v = to_internal(p);
    hipStream_t s = static_cast<hipStream_t>(stream);
    static_assert(sizeof(long long) == sizeof(int64_t), "int64 prefix sums");
    const long long *ck = reinterpret_cast<const long long *>(cu_k);
    if (r == R_PREFILL) {
        const size_t pneed = ds4idx::prefill_parts_workspace_bytes(v, k);
        if (pneed > 0 && (!workspace || !aligned(workspace, 256) || ws_bytes < pneed)) return DS4IDX_ERR_WORKSPACE;
        return launch_status(
            ds4idx::launch_mfma_select_varlen(v, cu_q, ck, Q, K, K_scale, W, k, idx, vals, workspace, s));
    }
    const size_t need = ds4idx::split_workspace_bytes(ds4idx::split_shape(v), k);
    if (!workspace || !aligned(workspace, 256) || ws_bytes < need) return DS4IDX_ERR_WORKSPACE;
    return launch_status(
        ds4idx::launch_split_select_varlen(v, cu_q, ck, Q, K, K_scale, W, k, idx, vals, workspace, s));
}

int ds4idx_select_qfp8(const ds4idx_problem *p, const void *Q8, const float *Q_scale, const void *K,
                       const float *K_scale, const float *W, int32_t k, int32_t *idx, float *vals, void *stream)
{
    if (!p || p->B < 1 || p->T < 1 || p->S < 1 || p->H < 1 || p->D < 1 || p->causal_offset < 0 ||
        p->causal_offset + (int64_t)p->T > (int64_t)p->S || p->q_dtype != DS4IDX_FP8_E4M3 ||
        p->k_dtype != DS4IDX_FP8_E4M3)
        return DS4IDX_ERR_INVALID_ARG;
    if (k < 1 || k > DS4IDX_MAX_TOPK) return DS4IDX_ERR_INVALID_ARG;
    if (!Q8 || !Q_scale || !K || !K_scale || !W || !idx || !aligned(Q8, 16) || !aligned(K, 16) ||
        !aligned(Q_scale, 4) || !aligned(K_scale, 4) || !aligned(W, 4) || !aligned(idx, 4) || (vals && !aligned(vals, 4)))
        return DS4IDX_ERR_INVALID_ARG;
    if (p->H != ds4idx::kMfmaH || p->D != ds4idx::kMfmaD || k > ds4idx::kMfmaMaxK || p->B > 65535)
        return DS4IDX_ERR_UNSUPPORTED;
    const Problem q = to_internal(p);
    return launch_status(ds4idx::launch_mfma_select_qfp8(q, Q8, Q_scale, K, K_scale, W, k, idx, vals,
                                                         static_cast<hipStream_t>(stream)));
}

int ds4idx_sparse_attention(const ds4idx_attn_problem *p, const void *Q, const void *KV,
                            const int32_t *idx, void *O, float *lse, void *stream)
{
    if (!p || p->B < 1 || p->T < 1 || p->S < 1 || p->H < 1 || p->topk < 1 || p->topk > DS4IDX_MAX_TOPK ||
        p->d_qk < 1 || p->d_v < 1 || p->d_v > p->d_qk || !std::isfinite(p->softmax_scale))
        return DS4IDX_ERR_INVALID_ARG;
    if (!Q || !KV || !idx || !O || !aligned(Q, 16) || !aligned(KV, 16) || !aligned(O, 16) || !aligned(idx, 4) ||
        (lse && !aligned(lse, 4)))
        return DS4IDX_ERR_INVALID_ARG;
    if (p->d_qk != ds4idx::kAttnDqk || p->d_v != ds4idx::kAttnDv || p->H % ds4idx::kAttnHeadTile != 0 ||
        p->H / ds4idx::kAttnHeadTile > 65535 || (int64_t)p->B * p->T > (int64_t)INT32_MAX)
        return DS4IDX_ERR_UNSUPPORTED;
    const ds4idx::AttnProblem a{p->B, p->T, p->S, p->H, p->topk, p->softmax_scale};
    return launch_status(ds4idx::launch_sparse_attention(a, Q, KV, idx, O, lse, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
