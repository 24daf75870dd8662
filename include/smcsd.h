/*
 * smcsd.h - C ABI of the MI355X (gfx950) SMC-SD verify / resample / KV pointer-exchange
 * library (libsmcsd.so).
 *
 * The method: Sequential Monte Carlo speculative decoding as described by the two
 * explainers of "Faster LLM Inference via Sequential Monte Carlo" (gist.science,
 * Chinese and Spanish pages).  Each round, a draft model extends N particles by K
 * tokens; the target model scores all of them in one batched pass and adds one bonus
 * token per particle; each particle's importance weight is updated with the
 * target/draft probability ratio; when the effective sample size (ESS) falls below a
 * threshold the population is resampled by weight, and the KV cache follows by
 * exchanging block pointers and reference counts, never copying KV data (methodology
 * section, "core flow" and "system optimisation design"; Spanish page, "Resumen
 * Tecnico" section 2).  The speculative-sampling notes ("Accelerating-Large-Language-
 * Model-Decoding-with-Speculative-Sampling", section 1 and section 4.2) define the
 * secondary SpS mode: modified rejection sampling on the same logits.
 *
 * Conventions for every entry point
 *   - Array arguments are DEVICE pointers owned by the caller; the library allocates
 *     nothing, keeps no state between calls and never synchronises the stream.  (The
 *     one value it keeps is a constant of the build: the streaming kernel's static LDS
 *     size, read once from the runtime to size the unused dynamic LDS that holds that
 *     kernel to four workgroups per compute unit.  smcsd_verify_static, for callers that
 *     cannot allocate, uses a scratch array inside the library instead of a workspace.)
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All work is
 *     enqueued on it, in call order.
 *   - Host-detectable argument errors return a negative code before anything is
 *     enqueued (SMCSD_EINVAL, SMCSD_EDTYPE, SMCSD_EWORKSPACE); a failed launch returns
 *     SMCSD_EHIP.  0 means the work was enqueued.
 *   - Conditions found on the device are OR'ed into the caller's int32 `status` word
 *     (SMCSD_ST_*), which the caller zeroes and reads after its own synchronisation.
 *     Kernels bounds-check every index they read from device memory (tokens,
 *     ancestors, block ids) and flag SMCSD_ST_BAD_INPUT instead of faulting.
 *   - Calls that share a workspace or state arrays must not overlap in time.
 *
 * Randomness (the pages name no generator): Philox4x32-10 (Salmon et al., SC'11) with
 * key = (seed low, seed high) and counter = (stream index, step low, step high, tag);
 * a uniform is (word >> 8) * 2^-24.  Tags: 1 bonus token (index = sequence g),
 * 2 resampling offset (index = prompt b), 3 | (k/4) << 8 SpS acceptance of draft k
 * (word k mod 4), 4 SpS final token, 5 | pos << 8 draft token at draft position pos
 * (index = row), 6 | (v/4) << 8 the race-mode clock of vocabulary entry v (word v mod 4,
 * index = sequence g; that clock uses (floor(word / 2^9) + 1/2) * 2^-23).  Results depend only
 * on (inputs, seed, step): runs are bit-reproducible and resumable.
 */
#ifndef SMCSD_H
#define SMCSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMCSD_VERSION 7

/* logits element type */
#define SMCSD_DTYPE_F32 0
#define SMCSD_DTYPE_BF16 1

/* verify mode */
#define SMCSD_MODE_SMC 0
#define SMCSD_MODE_SPS 1
#define SMCSD_MODE_SMC_RACE 2 /* SMC mode, bonus token by an exponential race */

/* host return codes */
#define SMCSD_OK 0
#define SMCSD_EINVAL (-1)
#define SMCSD_EDTYPE (-2)
#define SMCSD_EHIP (-3)
#define SMCSD_EWORKSPACE (-4)
#define SMCSD_ESCRATCH (-5) /* smcsd_verify_static: needs more than SMCSD_STATIC_SCRATCH_BYTES */

/* device status bits (sticky, OR'ed into *status) */
#define SMCSD_ST_NAN_INPUT 1          /* a NaN or +inf logit in a row that was read      */
#define SMCSD_ST_EMPTY_ROW 2          /* a row with no finite logit (all -inf)           */
#define SMCSD_ST_NOSPACE 4            /* the free stack ran out during a reservation      */
#define SMCSD_ST_DEGENERATE_WEIGHTS 8 /* a prompt whose weights are all zero or NaN       */
#define SMCSD_ST_BAD_INPUT 16         /* token, ancestor or block id out of range         */
#define SMCSD_ST_KV_INCONSISTENT 32   /* smcsd_kv_check found a violated invariant        */

/* workspace query ops */
#define SMCSD_OP_VERIFY_SMC 0
#define SMCSD_OP_VERIFY_SPS 1
#define SMCSD_OP_KV 2
#define SMCSD_OP_DRAFT 3
#define SMCSD_OP_KV_CHECK 4

/* kinds of violation counted by smcsd_kv_check */
#define SMCSD_KV_CHECK_KINDS 5

/* Library version (SMCSD_VERSION). */
int smcsd_version(void);

/* Static text for a host return code or a single device status bit. */
const char *smcsd_status_string(int code);

/*
 * Device workspace bytes for one call.  Workspaces are caller-owned device buffers whose
 * start must be 256-byte aligned (SMCSD_EWORKSPACE otherwise).
 *   SMCSD_OP_VERIFY_SMC / _SPS: B, N, K, V as passed to smcsd_verify (P ignored).
 *   SMCSD_OP_DRAFT: B = number of rows, N = 1, V as passed to smcsd_draft_sample.
 *   SMCSD_OP_KV_CHECK: the pool size P (B, N, K, V ignored); no initial contents needed.
 *   SMCSD_OP_KV: B, N and the pool size P (K, V ignored).  The KV workspace must be
 *   zero-filled before its first use and then passed, unmodified, to every later call
 *   with the same B, N and P: calls keep its contents consistent (it alternates two
 *   freed-block bitmaps and clears the one the previous call used).
 * Returns 0 for invalid sizes.
 */
size_t smcsd_workspace_bytes(int op, int B, int N, int K, int V, int64_t P);

/*
 * smcsd_verify - the Score, Bonus and Reweight steps of one SMC-SD round (SMC mode),
 * or the SpS modified-rejection verify (SpS mode), over B*N sequences.
 * Defining passages: SMC explainers, methodology "core flow" (score the K drafted
 * tokens of every particle in one batched target pass, add one bonus token per
 * sequence, reweight by the target/draft ratio; always K+1 tokens per round); the
 * speculative-sampling notes, section 1 (draft K, score in parallel, accept or
 * resample so the output follows the target) and section 4.2.
 *
 * Sequences and layout.  Output sequence g in [0, B*N) reads source sequence
 * src = g * seq_step (seq_step = 1 for SMC; seq_step = N_smc selects particle 0 of
 * each prompt for an SpS comparison on the same tensors).  Row k of src starts at
 *   target_logits + (src*(K+1) + k) * row_stride   (k = 0..K, element units)
 *   draft_logits  + (src*K     + k) * row_stride   (k = 0..K-1)
 * with V valid elements per row (row_stride >= V).  dtype = SMCSD_DTYPE_BF16 or
 * SMCSD_DTYPE_F32; pointers must be element-aligned (16-byte alignment is fastest).
 * draft_tokens [src, K] int32 in [0, V); lse_in (nullable) [src, 2K+1] fp32.
 *
 * Arithmetic.  z = logit / temperature.  Each row's log-normaliser
 * LSE = max z + ln sum exp(z - max z) is accumulated in fp32 in one streaming pass.
 *   logp_k = z^t_k[x_k] - LSE^t_k,  logq_k = z^d_k[x_k] - LSE^d_k   (k < K)
 * SMC mode: bonus = min{v : sum_{w<=v} softmax(z^t_K)_w > u}, u = U(seed; g, step,
 * tag 1); logp_K = its log-probability; then
 *   log_weights[g] += sum_{k<K} (alpha*logp_k - logq_k) + (alpha-1)*logp_K
 * (alpha = 1: the plain target/draft ratio; alpha != 1: power-sampling target
 * alpha*log p, not renormalised).  out_tokens[g] = (x_0..x_{K-1}, bonus),
 * out_num_tokens[g] = K+1.
 * SpS mode: keep x_k while r_k < p_k(x_k)/q_k(x_k) (r_k = U(seed; g, step, 3|(k/4)<<8,
 * word k mod 4)); at the first rejection k* draw from max(0, p - q) renormalised
 * (p if that residual is empty), else a bonus from p_K (u = U(seed; g, step, 4));
 * out_tokens[g] = accepted drafts then the drawn token, padded with -1;
 * out_num_tokens[g] = k*+1 (K+1 if all accepted); out_logp[g][K] = target
 * log-probability of the drawn token at its position; log_weights is not touched.
 * SMC race mode: SMC mode with the bonus drawn by an exponential race (the
 * exponential-races summary page, key design: token v finishes at E_v / p_v with
 * E_v ~ Exp(1), and the first to finish is a draw from p):
 *   bonus = argmax_v (z^t_K[v] - ln E_v),  E_v = -ln u_v,
 *   u_v = (floor(w / 2^9) + 1/2) * 2^-23,  w = word (v mod 4) of the Philox block with
 *   counter (g, step low, step high, 6 | (v div 4) << 8) and key (seed low, seed high);
 * equal keys go to the smaller v.  The keys are evaluated in fp32 during the LSE pass,
 * so the bonus row is read once; everything else is as in SMC mode.
 * If lse_in is given (SpS mode only) the LSE pass is skipped and lse_in is used.
 * If logq_in is given (SMC or SMC race mode) [src, K] fp32 - the draft's log-probabilities of
 * its own tokens, as smcsd_draft_sample emits them while drafting - the draft rows are
 * not read at all (draft_logits may be NULL): logq_k = logq_in[src][k], and the LSE
 * pass covers only the K+1 target rows (out_lse's draft entries are NaN).  The bytes
 * read per sequence fall from (2K+1)V to (K+1)V.
 *
 * Outputs (indexed by g): out_tokens [B*N, K+1] int32 (required); out_num_tokens
 * [B*N], out_logp [B*N, K+1], out_logq [B*N, K], out_lse [B*N, 2K+1] (target rows
 * 0..K then draft rows 0..K-1), all nullable.  log_weights [B*N] fp32 in/out
 * (required in the SMC modes).
 * Limits: 0 <= K <= 32, 1 <= V <= 2^24, temperature finite > 0, alpha finite.
 * B*N = 0 is a no-op.  workspace: smcsd_workspace_bytes(SMCSD_OP_VERIFY_SMC, ...) for
 * the SMC modes, SMCSD_OP_VERIFY_SPS for SpS.
 */
int smcsd_verify(const void *target_logits, const void *draft_logits, int dtype,
                 int64_t row_stride, int seq_step, const int32_t *draft_tokens, int B, int N,
                 int K, int V, float temperature, float alpha, int mode, uint64_t seed,
                 uint64_t step, const float *lse_in, const float *logq_in, float *log_weights,
                 int32_t *out_tokens, int32_t *out_num_tokens, float *out_logp, float *out_logq,
                 float *out_lse, int32_t *status, void *workspace, size_t workspace_bytes,
                 void *stream);

/*
 * smcsd_verify_static - smcsd_verify for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument; the kernels' scratch (per-tile (max, sum) partials, bonus slab sums,
 * race winners, SpS residual partials) is a device array inside the library of
 * SMCSD_STATIC_SCRATCH_BYTES, one copy per GPU, located on the first call on each device
 * and held until the process ends.  Arguments, layouts, outputs, status bits and limits are
 * those of smcsd_verify, whose results it reproduces bit for bit (the same kernels).
 * Returns SMCSD_ESCRATCH, before anything is enqueued, when the call needs more scratch
 * than the array holds, i.e. smcsd_workspace_bytes(SMCSD_OP_VERIFY_SMC or _SPS, B, N, K, V,
 * 0) > SMCSD_STATIC_SCRATCH_BYTES (the five reference shapes need at most 3 MB); SMCSD_EHIP
 * if the array cannot be located.  It allocates nothing and needs no clearing (each call
 * writes every scratch entry before reading it), but every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (two streams, two host threads) race,
 * and the caller must serialise them.
 */
#define SMCSD_STATIC_SCRATCH_BYTES (4u << 20)
int smcsd_verify_static(const void *target_logits, const void *draft_logits, int dtype,
                        int64_t row_stride, int seq_step, const int32_t *draft_tokens, int B,
                        int N, int K, int V, float temperature, float alpha, int mode,
                        uint64_t seed, uint64_t step, const float *lse_in, const float *logq_in,
                        float *log_weights, int32_t *out_tokens, int32_t *out_num_tokens,
                        float *out_logp, float *out_logq, float *out_lse, int32_t *status,
                        void *stream);

/*
 * smcsd_draft_sample - the draft side of the Extend step at one draft position: each
 * of n rows (one sequence's draft logits at position pos) draws its token from its own
 * tempered distribution and also yields that token's log-probability, which is what
 * the verify's reweighting needs from the draft (SMC explainers, methodology "core
 * flow": the draft model extends every particle by K tokens).  The draw is a reading:
 * x = min{v : sum_{w<=v} softmax(z)_w > u}, z = logit / temperature,
 * u = U(seed; r, step, 5 | pos << 8) for row r; out_logq[r] = z_x - LSE(z) (fp32
 * accumulation, as in smcsd_verify).  Passing these values as smcsd_verify's logq_in
 * lets the verify skip the draft rows.
 * Layout: draft_logits + r * row_stride (element units), V valid elements per row,
 * dtype bf16 or fp32, element-aligned.  out_tokens [n] int32 (-1 for a row with no
 * finite logit, which also sets EMPTY_ROW), out_logq [n] fp32 (nullable).
 * Limits: 1 <= V <= 2^24, 0 <= pos < 2^24, temperature finite > 0.  n = 0 is a
 * no-op.  workspace: smcsd_workspace_bytes(SMCSD_OP_DRAFT, n, 1, 0, V, 0).
 */
int smcsd_draft_sample(const void *draft_logits, int dtype, int64_t row_stride, int n, int V,
                       float temperature, uint64_t seed, uint64_t step, int pos,
                       int32_t *out_tokens, float *out_logq, int32_t *status, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * smcsd_resample - ESS and resampling per prompt (the Resample step: compute the
 * effective sample size every round and, when it is below the threshold, copy
 * high-weight particles and drop low-weight ones; SMC explainers, methodology
 * "core flow").  The ESS formula and the scheme are readings: with m = max_n lw,
 * w_n = exp(lw_n - m) in fp64, ESS = (sum w)^2 / sum w^2 clamped to [1, N];
 * prompt b resamples iff ESS < tau*N; systematic resampling with one offset
 * u0 = U(seed; b, step, tag 2): ancestors[b, i] = min{j : C_j > (i+u0)/N} with
 * C_j = sum_{i<=j} w_i / sum w (clamped to N-1, non-decreasing in i); the prompt's
 * log-weights are then reset to 0.  Otherwise ancestors[b, i] = i and log_weights
 * are unchanged.
 * Arrays: log_weights [B, N] fp32 in/out; ancestors [B, N] int32, ess [B] fp32,
 * resampled [B] int32 (0/1) out.  Limits: 1 <= N <= 1024, tau finite.
 * A prompt whose weights are all zero or NaN keeps identity ancestors, gets ess = 0
 * and sets SMCSD_ST_DEGENERATE_WEIGHTS.
 */
int smcsd_resample(float *log_weights, int B, int N, float tau, uint64_t seed, uint64_t step,
                   int32_t *ancestors, float *ess, int32_t *resampled, int32_t *status,
                   void *stream);

/*
 * smcsd_kv_reassign - the KV cache after resampling by pointer exchange and
 * reference counts, with prefixes shared across particles and no KV data copied
 * (SMC explainers, "system optimisation design": KV cache; Spanish page, cache
 * management).  Block-table rules (readings; the pages give only the principle):
 *
 * State: block_tables [B*N, M_cap] int32 block ids (-1 = unallocated); every sequence
 * has positions [0, seq_len) allocated in slots [0, ceil(seq_len/block_size)); slots
 * beyond hold -1.  refcounts [P] = number of table references per block; the free
 * stack is free_list[0 .. *free_top) with its top at index *free_top - 1.
 * Phase 1, prompts with resampled[b] != 0: c_j = #{i : ancestors[b,i] = j};
 * refcounts of every allocated block of old table j change by c_j - 1 (all increments
 * before any decrement); blocks reaching 0 are freed; new table i = old table
 * ancestors[b,i].  The freed blocks of the call are pushed in descending id order.
 * Phase 2, all prompts: reserve positions [seq_len, seq_len + reserve_tokens).  From
 * the post-phase-1 tables, a sequence whose partial tail block (slot
 * floor(seq_len/block_size) when seq_len mod block_size != 0) is also held by a
 * higher-index sequence of its prompt (the highest holder keeps the block) does
 * copy-on-write: it pops a
 * fresh block d, the old block loses one reference, and (old, d, seq_len mod
 * block_size) is appended to cow [B*N, 3] - the caller copies that many token
 * entries of KV data from old to d before writing the round.  Then every slot in
 * [ceil(seq_len/bs), ceil((seq_len+reserve_tokens)/bs)) pops a fresh block with
 * refcount 1.  Pops run in ascending (sequence, slot) order; when the stack is empty
 * the slot keeps its value (-1, or the shared tail) and SMCSD_ST_NOSPACE is set.
 * Indices read from memory are checked first (SMCSD_ST_BAD_INPUT, nothing faults): a
 * resampled prompt with an ancestor outside [0, N) is left unexchanged; a block id
 * outside [0, P) in an allocated slot of a resampled prompt's old tables (such as a
 * slot a NOSPACE call left at -1) changes no count; a tail block id >= P makes no
 * copy-on-write; a free-stack entry outside [0, P) leaves its slot as it was, and a
 * copy-on-write that pops one is listed with destination -1 and does nothing else.
 * *cow_count = number of copy-on-write entries written.
 * Call once with identity ancestors (resampled all 0) before the first round to
 * reserve its K+1 slots; after round t call with seq_len = tokens now held
 * (previous seq_len + K+1).
 * Limits: 1 <= N <= 1024; ceil((seq_len+reserve_tokens)/block_size) <= M_cap.
 * workspace: smcsd_workspace_bytes(SMCSD_OP_KV, B, N, 0, 0, P), zero-filled before
 * first use and kept, unmodified, between calls.
 */
int smcsd_kv_reassign(const int32_t *ancestors, const int32_t *resampled, int B, int N,
                      int32_t *block_tables, int M_cap, int block_size, int64_t seq_len,
                      int reserve_tokens, int32_t *refcounts, int32_t *free_list,
                      int32_t *free_top, int64_t P, int32_t *cow, int32_t *cow_count,
                      int32_t *status, void *workspace, size_t workspace_bytes, void *stream);

/*
 * smcsd_resample_kv_reassign - smcsd_resample followed by smcsd_kv_reassign, in one
 * launch fewer: the Resample step of the round (SMC explainers, methodology "core
 * flow") and the KV pointer exchange that follows it ("system optimisation design":
 * KV cache) run in the same per-prompt workgroup, which takes its prompt's ancestors
 * from on-chip memory.  Arguments, layouts, limits, outputs and status bits are those
 * of the two calls: log_weights [B, N] in/out, ancestors [B, N], ess [B] and
 * resampled [B] are written exactly as smcsd_resample writes them (the same bits), and
 * the block tables, refcounts, free stack and copy-on-write list end exactly as
 * smcsd_kv_reassign leaves them given those ancestors.  Limits: those of both calls
 * (1 <= N <= 1024, tau finite).  workspace: smcsd_workspace_bytes(SMCSD_OP_KV, B, N, 0,
 * 0, P), shared with smcsd_kv_reassign (the two may alternate on one workspace).
 */
int smcsd_resample_kv_reassign(float *log_weights, int B, int N, float tau, uint64_t seed,
                               uint64_t step, int32_t *ancestors, float *ess, int32_t *resampled,
                               int32_t *block_tables, int M_cap, int block_size, int64_t seq_len,
                               int reserve_tokens, int32_t *refcounts, int32_t *free_list,
                               int32_t *free_top, int64_t P, int32_t *cow, int32_t *cow_count,
                               int32_t *status, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * smcsd_step - one whole SMC-SD round on the batch: smcsd_verify (SMC or SMC race mode;
 * row_stride and the draft's optional log q as there, seq_step 1) followed by
 * smcsd_resample_kv_reassign, with the same outputs and the same bits as those two calls
 * (SMC explainers, methodology "core flow": Score, Bonus, Reweight, then Resample and the
 * KV pointer exchange of "system optimisation design").  It enqueues the two calls'
 * kernels in order on `stream` with one host call, for callers that run a whole round per
 * call; both workspaces stay separate, so a round can also be split into the two calls.
 * Arguments: those of smcsd_verify (log_weights [B, N] in/out; out_tokens required;
 * out_num_tokens, out_logp, out_logq, out_lse nullable) and of smcsd_resample_kv_reassign
 * (tau; ancestors [B, N], ess [B], resampled [B]; the KV state; seq_len is the length
 * after this round's K+1 tokens, as there); verify_workspace sized by
 * smcsd_workspace_bytes(SMCSD_OP_VERIFY_SMC, B, N, K, V, 0) and kv_workspace by
 * smcsd_workspace_bytes(SMCSD_OP_KV, B, N, 0, 0, P) (zero-filled before first use and kept,
 * shared with smcsd_kv_reassign and smcsd_resample_kv_reassign).  Limits, errors and status
 * bits: those of both calls; mode SMCSD_MODE_SPS is SMCSD_EINVAL.
 */
int smcsd_step(const void *target_logits, const void *draft_logits, int dtype, int64_t row_stride,
               const int32_t *draft_tokens, int B, int N, int K, int V, float temperature,
               float alpha, int mode, float tau, uint64_t seed, uint64_t step,
               const float *logq_in, float *log_weights, int32_t *out_tokens,
               int32_t *out_num_tokens, float *out_logp, float *out_logq, float *out_lse,
               int32_t *ancestors, float *ess, int32_t *resampled, int32_t *block_tables,
               int M_cap, int block_size, int64_t seq_len, int reserve_tokens, int32_t *refcounts,
               int32_t *free_list, int32_t *free_top, int64_t P, int32_t *cow, int32_t *cow_count,
               int32_t *status, void *verify_workspace, size_t verify_workspace_bytes,
               void *kv_workspace, size_t kv_workspace_bytes, void *stream);

/*
 * smcsd_kv_check - debugging check of the refcounted block-table state that
 * smcsd_kv_reassign, smcsd_resample_kv_reassign and smcsd_step maintain (SMC explainers,
 * "system optimisation design": KV blocks shared by pointer and released by reference
 * count; Spanish page, cache management).  It recounts everything from the arrays
 * themselves, independently of the exchange kernels, and counts violations per kind:
 *   violations[0]  blocks whose refcount differs from the number of allocated table
 *                  slots naming them;
 *   violations[1]  allocated table slots holding an id outside [0, P) other than the
 *                  -1 of a slot a NOSPACE call left unfilled;
 *   violations[2]  free-stack entries outside [0, P), extra occurrences of a block on
 *                  the stack, and a top outside [0, P] (then clamped);
 *   violations[3]  blocks on the free stack with a positive refcount;
 *   violations[4]  blocks with refcount <= 0 that are not on the free stack (leaked).
 * A consistent state has all five at 0: live and free blocks then partition the pool.
 * block_tables [S, M_cap] int32 with slots [0, slots) allocated in every row (after a
 * reassign call with seq_len L and reserve R: slots = ceil((L + R) / block_size));
 * refcounts [P], free_list [P], free_top [1] int32 as in smcsd_kv_reassign; all read
 * only.  violations [SMCSD_KV_CHECK_KINDS] int32 device output, overwritten (not
 * accumulated); SMCSD_ST_KV_INCONSISTENT is OR'ed into *status when any is nonzero.
 * workspace: smcsd_workspace_bytes(SMCSD_OP_KV_CHECK, 0, 0, 0, 0, P), 256-byte
 * aligned, any contents.  Limits: S >= 0, 0 <= slots <= M_cap, 1 <= P <= 2^31 - 1.
 * Five small launches; meant for tests and debug runs (the Python binding runs it after
 * every KV call when the environment variable SMCSD_DEBUG_CHECK is 1), not the timed path.
 */
int smcsd_kv_check(const int32_t *block_tables, int64_t S, int M_cap, int slots,
                   const int32_t *refcounts, const int32_t *free_list, const int32_t *free_top,
                   int64_t P, int32_t *violations, int32_t *status, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * smcsd_philox4x32_10 - the library's device Philox4x32-10 block function (SC'11),
 * exposed so its bit-exactness can be checked: out[i] = Philox(counters[i],
 * keys[i]) for i < n.  counters [n, 4], keys [n, 2], out [n, 4] uint32 device arrays.
 */
int smcsd_philox4x32_10(const uint32_t *counters, const uint32_t *keys, int n, uint32_t *out,
                        void *stream);

/*
 * smcsd_stream_read - a measurement aid, not a step of the method.  The verify's LSE pass
 * is one streaming read of the logits with a few operations per element (decoding is
 * bound by memory bandwidth: SMC explainers, problem statement), so its speed of light is
 * the rate at which this GPU streams reads from HBM.  This call reads each 16-byte word of
 * [p, p + bytes) once, with the LSE pass's load instruction (16-byte nontemporal buffer
 * loads), one workgroup per contiguous tile of SMCSD_STREAM_READ_TILE_BYTES, and writes
 * tile_xor[b] = the XOR of the 32-bit words of tile b (bytes [b*T, min(bytes, (b+1)*T)),
 * T the tile size), for b < ceil(bytes / T): a device uint32 array, overwritten.  bytes
 * divided by the time of the call is the achievable read rate that the LSE pass's rate is
 * compared with.  p: device memory, 16-byte aligned; bytes a multiple of 16,
 * 0 <= bytes <= SMCSD_STREAM_READ_MAX_BYTES (bytes = 0: nothing is read or written, and p
 * and tile_xor may be NULL); otherwise SMCSD_EINVAL before any launch.  One launch.
 */
#define SMCSD_STREAM_READ_TILE_BYTES 131072
#define SMCSD_STREAM_READ_MAX_BYTES (1LL << 40)
int smcsd_stream_read(const void *p, int64_t bytes, uint32_t *tile_xor, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SMCSD_H */
