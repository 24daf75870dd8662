// capi.hip - extern "C" entry points of libsmcsd.so: argument validation, dtype
// dispatch and launch.  Declarations and the full contract are in include/smcsd.h.
#include <cmath>
#include <mutex>

#include "../../include/smcsd.h"
#include "internal.hpp"
#include "kv_layout.hpp"

using namespace smcsd;

namespace {

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline int hip_rc(hipError_t e) { return e == hipSuccess ? SMCSD_OK : SMCSD_EHIP; }

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

int smcsd_version(void) { return SMCSD_VERSION; }

const char *smcsd_status_string(int code) {
  switch (code) {
    case SMCSD_OK: return "ok";
    case SMCSD_EINVAL: return "invalid argument";
    case SMCSD_EDTYPE: return "unsupported dtype";
    case SMCSD_EHIP: return "HIP launch error";
    case SMCSD_EWORKSPACE: return "workspace too small or missing";
    case SMCSD_ESCRATCH: return "call needs more scratch than the static array holds";
    case SMCSD_ST_NAN_INPUT: return "NaN or +inf logit";
    case SMCSD_ST_EMPTY_ROW: return "row with no finite logit";
    case SMCSD_ST_NOSPACE: return "block pool exhausted";
    case SMCSD_ST_DEGENERATE_WEIGHTS: return "all particle weights zero or NaN";
    case SMCSD_ST_BAD_INPUT: return "token, ancestor or block id out of range";
    case SMCSD_ST_KV_INCONSISTENT: return "block tables, refcounts and free stack disagree";
    default: return "unknown code";
  }
}

size_t smcsd_workspace_bytes(int op, int B, int N, int K, int V, int64_t P) {
  if (B < 0 || N < 0) return 0;
  const int64_t S = (int64_t)B * N;
  if (op == SMCSD_OP_VERIFY_SMC || op == SMCSD_OP_VERIFY_SPS) {
    if (K < 0 || K > kMaxK || V < 1 || V > kMaxV) return 0;
    return verify_ws_layout(S, K, V, op == SMCSD_OP_VERIFY_SPS ? 1 : 0).total;
  }
  if (op == SMCSD_OP_DRAFT) {
    if (V < 1 || V > kMaxV) return 0;
    return verify_ws_layout(S, 0, V, 0).total;
  }
  if (op == SMCSD_OP_KV) {
    if (P < 1) return 0;
    return kv_ws_layout(S, P).total;
  }
  if (op == SMCSD_OP_KV_CHECK) {
    if (P < 1 || P > INT32_MAX) return 0;
    return kv_check_ws_bytes(P);
  }
  return 0;
}

}  // extern "C"

namespace {

// The verify's scratch for callers that cannot allocate: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never uses the array's name as an
// address: each device's copy is found once with hipGetSymbolAddress and kept.
constexpr size_t kStaticScratchBytes = SMCSD_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's copy of the array (looked up on its first use on that device).
int static_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SMCSD_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SMCSD_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SMCSD_OK;
}

// smcsd_verify with the workspace either given (static_ws = false) or the library's array.
int verify_impl(const void *target_logits, const void *draft_logits, int dtype,
                int64_t row_stride, int seq_step, const int32_t *draft_tokens, int B, int N, int K,
                int V, float temperature, float alpha, int mode, uint64_t seed, uint64_t step,
                const float *lse_in, const float *logq_in, float *log_weights,
                int32_t *out_tokens, int32_t *out_num_tokens, float *out_logp, float *out_logq,
                float *out_lse, int32_t *status, void *workspace, size_t workspace_bytes,
                bool static_ws, void *stream) {
  if (dtype != SMCSD_DTYPE_F32 && dtype != SMCSD_DTYPE_BF16) return SMCSD_EDTYPE;
  if (mode != SMCSD_MODE_SMC && mode != SMCSD_MODE_SPS && mode != SMCSD_MODE_SMC_RACE)
    return SMCSD_EINVAL;
  const bool smc = mode != SMCSD_MODE_SPS;
  if (B < 0 || N < 0 || K < 0 || K > kMaxK || V < 1 || V > kMaxV || seq_step < 1)
    return SMCSD_EINVAL;
  if (row_stride < V) return SMCSD_EINVAL;
  if (!(temperature > 0.0f) || !std::isfinite(temperature) || !std::isfinite(alpha))
    return SMCSD_EINVAL;
  const int64_t S = (int64_t)B * N;
  if (S == 0) return SMCSD_OK;
  if (S > INT32_MAX / 2) return SMCSD_EINVAL;
  const size_t esz = dtype == SMCSD_DTYPE_BF16 ? 2 : 4;
  if (!target_logits || !aligned(target_logits, esz)) return SMCSD_EINVAL;
  if (logq_in && !smc) return SMCSD_EINVAL;
  if (K > 0 && (!draft_tokens || (!logq_in && (!draft_logits || !aligned(draft_logits, esz)))))
    return SMCSD_EINVAL;
  if (!out_tokens || !status) return SMCSD_EINVAL;
  if (smc && (!log_weights || lse_in)) return SMCSD_EINVAL;
  const size_t need = verify_ws_layout(S, K, V, mode == SMCSD_MODE_SPS ? 1 : 0).total;
  if (static_ws) {
    if (need > kStaticScratchBytes) return SMCSD_ESCRATCH;
    const int rc = static_scratch(&workspace);
    if (rc != SMCSD_OK) return rc;
    workspace_bytes = kStaticScratchBytes;
  }
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return SMCSD_EWORKSPACE;

  VerifyArgs a{};
  a.tgt = target_logits;
  a.drf = draft_logits;
  a.dtype = dtype;
  a.row_stride = row_stride;
  a.seq_step = seq_step;
  a.draft_tokens = draft_tokens;
  a.nseq = (int)S;
  a.K = K;
  a.V = V;
  a.c = (float)(1.4426950408889634073599246810018921 / (double)temperature);
  a.alpha = alpha;
  a.mode = mode;
  a.seed = seed;
  a.step = step;
  a.lse_in = lse_in;
  a.logq_in = logq_in;
  a.bonus_tag = 1u;
  a.log_weights = log_weights;
  a.out_tokens = out_tokens;
  a.out_num_tokens = out_num_tokens;
  a.out_logp = out_logp;
  a.out_logq = out_logq;
  a.out_lse = out_lse;
  a.status = status;
  a.ws = static_cast<char *>(workspace);
  a.stream = as_stream(stream);
  return hip_rc(launch_verify(a));
}

}  // namespace

extern "C" {

int smcsd_verify(const void *target_logits, const void *draft_logits, int dtype,
                 int64_t row_stride, int seq_step, const int32_t *draft_tokens, int B, int N,
                 int K, int V, float temperature, float alpha, int mode, uint64_t seed,
                 uint64_t step, const float *lse_in, const float *logq_in, float *log_weights,
                 int32_t *out_tokens, int32_t *out_num_tokens, float *out_logp, float *out_logq,
                 float *out_lse, int32_t *status, void *workspace, size_t workspace_bytes,
                 void *stream) {
  return verify_impl(target_logits, draft_logits, dtype, row_stride, seq_step, draft_tokens, B,
                     N, K, V, temperature, alpha, mode, seed, step, lse_in, logq_in, log_weights,
                     out_tokens, out_num_tokens, out_logp, out_logq, out_lse, status, workspace,
                     workspace_bytes, false, stream);
}

int smcsd_verify_static(const void *target_logits, const void *draft_logits, int dtype,
                        int64_t row_stride, int seq_step, const int32_t *draft_tokens, int B,
                        int N, int K, int V, float temperature, float alpha, int mode,
                        uint64_t seed, uint64_t step, const float *lse_in, const float *logq_in,
                        float *log_weights, int32_t *out_tokens, int32_t *out_num_tokens,
                        float *out_logp, float *out_logq, float *out_lse, int32_t *status,
                        void *stream) {
  return verify_impl(target_logits, draft_logits, dtype, row_stride, seq_step, draft_tokens, B,
                     N, K, V, temperature, alpha, mode, seed, step, lse_in, logq_in, log_weights,
                     out_tokens, out_num_tokens, out_logp, out_logq, out_lse, status, nullptr, 0,
                     true, stream);
}

int smcsd_draft_sample(const void *draft_logits, int dtype, int64_t row_stride, int n, int V,
                       float temperature, uint64_t seed, uint64_t step, int pos,
                       int32_t *out_tokens, float *out_logq, int32_t *status, void *workspace,
                       size_t workspace_bytes, void *stream) {
  if (dtype != SMCSD_DTYPE_F32 && dtype != SMCSD_DTYPE_BF16) return SMCSD_EDTYPE;
  if (n < 0 || V < 1 || V > kMaxV || row_stride < V || pos < 0 || pos >= (1 << 24))
    return SMCSD_EINVAL;
  if (!(temperature > 0.0f) || !std::isfinite(temperature)) return SMCSD_EINVAL;
  if (n == 0) return SMCSD_OK;
  const size_t esz = dtype == SMCSD_DTYPE_BF16 ? 2 : 4;
  if (!draft_logits || !aligned(draft_logits, esz) || !out_tokens || !status) return SMCSD_EINVAL;
  const size_t need = verify_ws_layout(n, 0, V, 0).total;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return SMCSD_EWORKSPACE;
  // the row-K draw of a verify with K = 0 over the draft rows, with the draft's RNG tag
  VerifyArgs a{};
  a.tgt = draft_logits;
  a.drf = nullptr;
  a.dtype = dtype;
  a.row_stride = row_stride;
  a.seq_step = 1;
  a.draft_tokens = nullptr;
  a.nseq = n;
  a.K = 0;
  a.V = V;
  a.c = (float)(1.4426950408889634073599246810018921 / (double)temperature);
  a.alpha = 1.0f;
  a.mode = SMCSD_MODE_SMC;
  a.seed = seed;
  a.step = step;
  a.log_weights = nullptr;
  a.out_tokens = out_tokens;
  a.out_logp = out_logq;
  a.status = status;
  a.ws = static_cast<char *>(workspace);
  a.stream = as_stream(stream);
  a.bonus_tag = 5u | ((uint32_t)pos << 8);
  return hip_rc(launch_verify(a));
}

int smcsd_resample(float *log_weights, int B, int N, float tau, uint64_t seed, uint64_t step,
                   int32_t *ancestors, float *ess, int32_t *resampled, int32_t *status,
                   void *stream) {
  if (B < 0 || N < 1 || N > kMaxN || !std::isfinite(tau)) return SMCSD_EINVAL;
  if (B == 0) return SMCSD_OK;
  if (!log_weights || !ancestors || !ess || !resampled || !status) return SMCSD_EINVAL;
  return hip_rc(launch_resample(log_weights, B, N, tau, seed, step, ancestors, ess, resampled,
                                status, as_stream(stream)));
}

// Host checks of a KV reassign call (SMCSD_OK to go ahead, 1 for an empty batch).
static int kv_check(int B, int N, const int32_t *block_tables, int M_cap, int block_size,
                    int64_t seq_len, int reserve_tokens, const int32_t *refcounts,
                    const int32_t *free_list, const int32_t *free_top, int64_t P, const int32_t *cow,
                    const int32_t *cow_count, const int32_t *status, const void *workspace,
                    size_t workspace_bytes) {
  if (B < 0 || N < 1 || N > kMaxN || M_cap < 1 || block_size < 1 || seq_len < 0 ||
      reserve_tokens < 0 || P < 1 || P > INT32_MAX)
    return SMCSD_EINVAL;
  if (ceil_div(seq_len + reserve_tokens, block_size) > M_cap) return SMCSD_EINVAL;
  if (B == 0) return 1;
  if ((int64_t)B * N * M_cap >= INT32_MAX) return SMCSD_EINVAL;  // 32-bit table indexing
  // one exchange workgroup per prompt part: the dispatch must stay under 2^32 threads
  const KvSplit ks = kv_split(N, (int)ceil_div(seq_len, block_size), (int)(seq_len % block_size));
  if ((int64_t)B * ks.parts * kKvThreads > (int64_t)0xFFFFFFFF) return SMCSD_EINVAL;
  if (!block_tables || !refcounts || !free_list || !free_top || !cow || !cow_count || !status)
    return SMCSD_EINVAL;
  const size_t need = kv_ws_layout((int64_t)B * N, P).total;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return SMCSD_EWORKSPACE;
  return SMCSD_OK;
}

int smcsd_kv_reassign(const int32_t *ancestors, const int32_t *resampled, int B, int N,
                      int32_t *block_tables, int M_cap, int block_size, int64_t seq_len,
                      int reserve_tokens, int32_t *refcounts, int32_t *free_list,
                      int32_t *free_top, int64_t P, int32_t *cow, int32_t *cow_count,
                      int32_t *status, void *workspace, size_t workspace_bytes, void *stream) {
  const int chk = kv_check(B, N, block_tables, M_cap, block_size, seq_len, reserve_tokens,
                           refcounts, free_list, free_top, P, cow, cow_count, status, workspace,
                           workspace_bytes);
  if (chk == 1) return SMCSD_OK;
  if (chk != SMCSD_OK) return chk;
  if (!ancestors || !resampled) return SMCSD_EINVAL;
  const FusedResample none{};
  return hip_rc(launch_kv(ancestors, resampled, none, B, N, block_tables, M_cap, block_size,
                          seq_len, reserve_tokens, refcounts, free_list, free_top, P, cow,
                          cow_count, status, static_cast<char *>(workspace), as_stream(stream)));
}

int smcsd_resample_kv_reassign(float *log_weights, int B, int N, float tau, uint64_t seed,
                               uint64_t step, int32_t *ancestors, float *ess, int32_t *resampled,
                               int32_t *block_tables, int M_cap, int block_size, int64_t seq_len,
                               int reserve_tokens, int32_t *refcounts, int32_t *free_list,
                               int32_t *free_top, int64_t P, int32_t *cow, int32_t *cow_count,
                               int32_t *status, void *workspace, size_t workspace_bytes,
                               void *stream) {
  if (!std::isfinite(tau)) return SMCSD_EINVAL;
  const int chk = kv_check(B, N, block_tables, M_cap, block_size, seq_len, reserve_tokens,
                           refcounts, free_list, free_top, P, cow, cow_count, status, workspace,
                           workspace_bytes);
  if (chk == 1) return SMCSD_OK;
  if (chk != SMCSD_OK) return chk;
  if (!log_weights || !ancestors || !ess || !resampled) return SMCSD_EINVAL;
  const FusedResample fr{log_weights, tau, seed, step, ancestors, ess, resampled};
  return hip_rc(launch_kv(nullptr, nullptr, fr, B, N, block_tables, M_cap, block_size, seq_len,
                          reserve_tokens, refcounts, free_list, free_top, P, cow, cow_count,
                          status, static_cast<char *>(workspace), as_stream(stream)));
}

int smcsd_step(const void *target_logits, const void *draft_logits, int dtype, int64_t row_stride,
               const int32_t *draft_tokens, int B, int N, int K, int V, float temperature,
               float alpha, int mode, float tau, uint64_t seed, uint64_t step,
               const float *logq_in, float *log_weights, int32_t *out_tokens,
               int32_t *out_num_tokens, float *out_logp, float *out_logq, float *out_lse,
               int32_t *ancestors, float *ess, int32_t *resampled, int32_t *block_tables,
               int M_cap, int block_size, int64_t seq_len, int reserve_tokens, int32_t *refcounts,
               int32_t *free_list, int32_t *free_top, int64_t P, int32_t *cow, int32_t *cow_count,
               int32_t *status, void *verify_workspace, size_t verify_workspace_bytes,
               void *kv_workspace, size_t kv_workspace_bytes, void *stream) {
  // the checks of smcsd_verify (SMC modes) and of smcsd_resample_kv_reassign
  if (dtype != SMCSD_DTYPE_F32 && dtype != SMCSD_DTYPE_BF16) return SMCSD_EDTYPE;
  if (mode != SMCSD_MODE_SMC && mode != SMCSD_MODE_SMC_RACE) return SMCSD_EINVAL;
  if (B < 0 || N < 1 || N > kMaxN || K < 0 || K > kMaxK || V < 1 || V > kMaxV) return SMCSD_EINVAL;
  if (row_stride < V) return SMCSD_EINVAL;
  if (!(temperature > 0.0f) || !std::isfinite(temperature) || !std::isfinite(alpha) ||
      !std::isfinite(tau))
    return SMCSD_EINVAL;
  const int chk = kv_check(B, N, block_tables, M_cap, block_size, seq_len, reserve_tokens,
                           refcounts, free_list, free_top, P, cow, cow_count, status, kv_workspace,
                           kv_workspace_bytes);
  if (chk == 1) return SMCSD_OK;
  if (chk != SMCSD_OK) return chk;
  const int64_t S = (int64_t)B * N;
  if (S > INT32_MAX / 2) return SMCSD_EINVAL;
  const size_t esz = dtype == SMCSD_DTYPE_BF16 ? 2 : 4;
  if (!target_logits || !aligned(target_logits, esz)) return SMCSD_EINVAL;
  if (K > 0 && (!draft_tokens || (!logq_in && (!draft_logits || !aligned(draft_logits, esz)))))
    return SMCSD_EINVAL;
  if (!out_tokens || !log_weights || !ancestors || !ess || !resampled) return SMCSD_EINVAL;
  const size_t need = verify_ws_layout(S, K, V, 0).total;
  if (!verify_workspace || !aligned(verify_workspace, 256) || verify_workspace_bytes < need)
    return SMCSD_EWORKSPACE;

  VerifyArgs a{};
  a.tgt = target_logits;
  a.drf = draft_logits;
  a.dtype = dtype;
  a.row_stride = row_stride;
  a.seq_step = 1;
  a.draft_tokens = draft_tokens;
  a.nseq = (int)S;
  a.K = K;
  a.V = V;
  a.c = (float)(1.4426950408889634073599246810018921 / (double)temperature);
  a.alpha = alpha;
  a.mode = mode;
  a.seed = seed;
  a.step = step;
  a.logq_in = logq_in;
  a.bonus_tag = 1u;
  a.log_weights = log_weights;
  a.out_tokens = out_tokens;
  a.out_num_tokens = out_num_tokens;
  a.out_logp = out_logp;
  a.out_logq = out_logq;
  a.out_lse = out_lse;
  a.status = status;
  a.ws = static_cast<char *>(verify_workspace);
  a.stream = as_stream(stream);
  // The verify's kernels, then the resample + exchange kernels on the same stream: the
  // latter read the log-weights the verify wrote.
  const hipError_t e = launch_verify(a);
  if (e != hipSuccess) return hip_rc(e);
  const FusedResample fr{log_weights, tau, seed, step, ancestors, ess, resampled};
  return hip_rc(launch_kv(nullptr, nullptr, fr, B, N, block_tables, M_cap, block_size, seq_len,
                          reserve_tokens, refcounts, free_list, free_top, P, cow, cow_count, status,
                          static_cast<char *>(kv_workspace), as_stream(stream)));
}

int smcsd_kv_check(const int32_t *block_tables, int64_t S, int M_cap, int slots,
                   const int32_t *refcounts, const int32_t *free_list, const int32_t *free_top,
                   int64_t P, int32_t *violations, int32_t *status, void *workspace,
                   size_t workspace_bytes, void *stream) {
  if (S < 0 || M_cap < 1 || slots < 0 || slots > M_cap || P < 1 || P > INT32_MAX)
    return SMCSD_EINVAL;
  if ((S > 0 && !block_tables) || !refcounts || !free_list || !free_top || !violations || !status)
    return SMCSD_EINVAL;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < kv_check_ws_bytes(P))
    return SMCSD_EWORKSPACE;
  return hip_rc(launch_kv_check(block_tables, S, M_cap, slots, refcounts, free_list, free_top, P,
                                violations, status, static_cast<char *>(workspace),
                                as_stream(stream)));
}

int smcsd_stream_read(const void *p, int64_t bytes, uint32_t *tile_xor, void *stream) {
  if (bytes < 0 || bytes > SMCSD_STREAM_READ_MAX_BYTES || (bytes & 15)) return SMCSD_EINVAL;
  if (bytes == 0) return SMCSD_OK;
  if (!p || !aligned(p, 16) || !tile_xor) return SMCSD_EINVAL;
  return hip_rc(launch_stream_read(p, bytes, tile_xor, as_stream(stream)));
}

int smcsd_philox4x32_10(const uint32_t *counters, const uint32_t *keys, int n, uint32_t *out,
                        void *stream) {
  if (n < 0) return SMCSD_EINVAL;
  if (n == 0) return SMCSD_OK;
  if (!counters || !keys || !out) return SMCSD_EINVAL;
  return hip_rc(launch_philox(counters, keys, n, out, as_stream(stream)));
}

}  // extern "C"
