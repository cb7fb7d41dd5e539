/*
 * dsa.h - C ABI of the DeepSeek Sparse Attention (DSA) hot path on AMD Instinct MI355X (gfx950).
 *
 * The method (DeepSeek-V3.2-Exp summary page, section "Method"; AMD "MI355X GPUs Power
 * DeepSeek-V3.2-Exp" article, sections "Lightning Indexer" and "Fine-Grained Token Selection"):
 *   1. a lightning indexer scores every causally visible key s of query token t,
 *        I[t,s] = sum_j w[t,j] * ReLU(q_I[t,j] . k_I[s]),  H_I heads, FP8 inputs;
 *   2. the top-k (k = 2048 in the model) keys per query are selected;
 *   3. MLA attention in MQA mode (one latent KV row shared by all query heads of a token)
 *      runs over only the selected rows.
 *
 * Conventions shared by every call
 *  - Pointers are device memory owned by the caller (hipMalloc / framework tensors), unless a
 *    parameter says otherwise.  The library allocates no device memory, keeps no pointer after a
 *    call returns and never synchronises: work is enqueued on `stream`; the caller keeps every
 *    buffer alive until that work completes.
 *  - Tensors are dense row-major.  FP8 means OCP E4M3 ("e4m3fn": bias 7, max 448, no infinity)
 *    passed as uint8 codes; bf16 is passed as uint16 bit patterns; scales are fp32, one per row
 *    of the last dimension, positive.
 *  - Causality: query row t sits at absolute position q_start + t and sees keys
 *    0 .. n_t - 1 with n_t = min(S, q_start + t + 1) (its own position included).
 *  - Base pointers must be 16-byte aligned.  Argument errors are detected on the host before
 *    anything is enqueued (no partial work) and return DSA_ERR_INVALID_ARGUMENT, or
 *    DSA_ERR_UNSUPPORTED for shapes outside the compiled set, or DSA_ERR_WORKSPACE_TOO_SMALL.
 *    Launch failures return DSA_ERR_HIP.  Faults inside kernels surface at the caller's next
 *    synchronisation.  dsa_last_error() gives a thread-local message for the last failing call.
 *  - T == 0 (or B == 0) is a valid no-op.
 *  - With the environment variable DSA_TRACE set (non-empty, not "0"), every kernel launch writes
 *    one line to stderr (kernel, grid, block, dynamic LDS, stream), and the fused calls one line
 *    with the workspace size given and used.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 2

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1,
  DSA_ERR_UNSUPPORTED = 2,
  DSA_ERR_WORKSPACE_TOO_SMALL = 3,
  DSA_ERR_HIP = 4
} dsa_status_t;

const char *dsa_status_string(dsa_status_t s);
/* Message of the last failing call on this host thread ("" if none). */
const char *dsa_last_error(void);
int dsa_abi_version(void);

/*
 * Stage timing, a profiling aid outside the method: after dsa_profile_begin(events, capacity),
 * every kernel that a dsa_* call made on this host thread enqueues records events[i] (i = 0, 1,
 * ... in launch order; caller-created hipEvent_t, timing enabled) on the call's stream right after
 * the kernel, until capacity events are used or dsa_profile_end() is called, which stops the
 * recording and returns the number recorded.  With an event recorded on the stream before the
 * call, consecutive events bracket each kernel of a fused call.  dsa_profile_kernel_name(i)
 * names the kernel behind events[i] of the last recording ("" out of range; the string is
 * static).  begin returns DSA_ERR_INVALID_ARGUMENT for a NULL array or capacity < 1.
 */
dsa_status_t dsa_profile_begin(hipEvent_t *events, int32_t capacity);
int32_t dsa_profile_end(void);
const char *dsa_profile_kernel_name(int32_t i);

/*
 * Lightning-indexer scores (summary page, "Method"; AMD article, "Lightning Indexer"):
 *   logits[t][s] = sum_j w[t][j] * max(0, (q_scale[t][j] dec(q8[t][j][:])) . (k_scale[s] dec(k8[s][:])))
 * for s < n_t.  Entries s >= n_t of each logits row are not written.
 *   q8 [T][H_I][D_I] u8, q_scale [T][H_I] f32, w [T][H_I] f32 (used as given, any sign),
 *   k8 [S][D_I] u8, k_scale [S] f32, logits [T][ld_logits] f32 with ld_logits >= S and a
 *   multiple of 4.  Supported: 1 <= H_I <= 64, D_I in {32, 64, 96, 128}, T <= 1,048,576 per call
 *   (16-row query tiles on the launch grid's second dimension, which the GPU caps at 65,536; more
 *   rows return DSA_ERR_UNSUPPORTED and are split by the caller).
 */
dsa_status_t dsa_indexer_logits(const uint8_t *q8, const float *q_scale, const float *w,
                                const uint8_t *k8, const float *k_scale, int64_t T, int64_t S,
                                int32_t H_I, int32_t D_I, int64_t q_start, float *logits,
                                int64_t ld_logits, hipStream_t stream);

/*
 * Per-query top-k (AMD article, "Fine-Grained Token Selection"): indices[t][0 .. m) with
 * m = min(k, n_t) are the key indices of the m largest logits[t][0 .. n_t) (finite scores;
 * -0.0 equals +0.0; equal scores go to the lower index), every index above the k-th score
 * first in ascending order, then the selected ties in ascending order (rows with n_t <= k list
 * 0 .. n_t - 1); indices[t][m .. k) = -1.
 * The order is deterministic.  Rows longer than 32768 need a workspace of
 * dsa_topk_workspace_size() bytes (0 otherwise).  Supported: 1 <= k <= 2048 (larger k up to
 * 32768 when S <= 32768).
 */
size_t dsa_topk_workspace_size(int64_t T, int64_t S, int32_t k);
dsa_status_t dsa_topk(const float *logits, int64_t ld_logits, int64_t T, int64_t S, int64_t q_start,
                      int32_t k, int32_t *indices, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * Allocation-free top-k, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same selection, order and
 * arguments as dsa_topk, without a workspace.  Rows longer than 32768 keep their per-chunk
 * candidates in a file-scope device array of the library, DSA_TOPK_NOALLOC_SCRATCH_BYTES (32 MiB)
 * per GPU, held until the process ends; a call whose dsa_topk_workspace_size(T, S, k) exceeds it
 * (e.g. more than 512 rows of 131072 scores at k = 2048) returns DSA_ERR_UNSUPPORTED before
 * anything is enqueued.  The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (concurrent streams or host threads) race and must be
 * serialised by the caller.
 */
#define DSA_TOPK_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
dsa_status_t dsa_topk_noalloc(const float *logits, int64_t ld_logits, int64_t T, int64_t S, int64_t q_start,
                              int32_t k, int32_t *indices, hipStream_t stream);

/*
 * Sparse MLA forward, MQA mode (summary page, "Method"): for query row t, head h and the valid
 * entries i of indices[t] (0 <= idx < n_t; anything else, including -1, is skipped; duplicates
 * count with multiplicity):
 *   z_i = sm_scale * q[t][h][:] . kv[idx_i][:],   out[t][h][:] = sum_i softmax(z)_i kv[idx_i][:D_v],
 *   lse[t][h] = log sum_i exp(z_i)   (natural log; -inf and out = 0 for a row with no valid entry).
 *   q [T][H][D_qk] bf16, kv [S][D_qk] bf16 (K = all D_qk columns, V = the first D_v),
 *   indices [T][k] i32, out [T][H][D_v] bf16, out_f32 [T][H][D_v] f32 (optional, NULL to skip),
 *   lse [T][H] f32 (optional).  Probabilities are rounded to fp16 for the P.V product and V is
 *   converted bf16 -> fp16, exact for |v| in [2^-17, 65504] (precondition |v| <= 65504).
 *   Supported: (D_qk, D_v) in {(576, 512), (80, 64)}, 1 <= H <= 128, 1 <= k <= 2048.
 *   Workspace (device, 256-byte aligned): NULL runs the bf16-staged kernel.  Non-NULL, with
 *   dsa_sparse_mla_workspace_size() bytes (DSA_ERR_WORKSPACE_TOO_SMALL below that), selects fp16
 *   staging where the dims have it ((576, 512); the size is 0 and the workspace unused otherwise):
 *   the S latent rows are first converted to fp16 in the workspace (round to nearest even), q is
 *   converted as it is loaded, and the scores come from fp16 products — the same products while
 *   every q and kv value has |x| in [2^-17, 65504] (precondition |q|, |kv| <= 65504; smaller
 *   magnitudes round to fp16's 2^-24 grid).  The two stagings agree to the tolerance of the fp32
 *   accumulation, not bit for bit.  The workspace holds nothing the caller reads.
 */
size_t dsa_sparse_mla_workspace_size(int64_t T, int64_t S, int32_t H, int32_t D_qk, int32_t D_v, int32_t k);
dsa_status_t dsa_sparse_mla_fwd(const uint16_t *q, const uint16_t *kv, const int32_t *indices,
                                int64_t T, int64_t S, int32_t H, int32_t D_qk, int32_t D_v, int32_t k,
                                int64_t q_start, float sm_scale, uint16_t *out, float *out_f32,
                                float *lse, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Sparse MLA backward (summary page, "Method": in the sparse training stage the main model trains
 * with top-k selection on, its attention reading only the listed rows; AMD article, "Training
 * Approach", sparse stage).  Gradients of a loss L through dsa_sparse_mla_fwd on the same lists,
 * given dout = dL/dout.  For query row t, head h and the valid entries i of indices[t] (as in the
 * forward: 0 <= idx_i < n_t, duplicates with multiplicity), p_i = exp(z_i - lse[t][h]):
 *   dp_i = dout[t][h] . v_i,   D = sum_i p_i dp_i  (= dout[t][h] . out[t][h]),   ds_i = p_i (dp_i - D),
 *   dq[t][h][:] = sm_scale sum_i ds_i k_i,
 *   dkv[s][:]   = sum over (t, h, i) with idx_i = s of  sm_scale ds_i q[t][h][:]  (all D_qk columns)
 *                 + p_i dout[t][h][:]  (the first D_v columns).
 *   q, kv, indices, sm_scale, q_start as in the forward; lse [T][H] f32 is the forward's output on
 *   the same inputs (D is summed from p and dp here, not taken from a rounded forward output);
 *   dout [T][H][D_v] bf16; dq [T][H][D_qk] f32 and dkv [S][D_qk] f32 are outputs (every entry
 *   written; keys no list selects get 0).  Workspace: dsa_sparse_mla_bwd_workspace_size(T, S, H, k)
 *   bytes, the buffers of one chunk of up to 512 query rows (fp16 ds and p per head and entry, one
 *   fp32 576-wide dkv contribution per entry, a key-to-entry map over S keys: about 3 GB at 512 rows,
 *   H = 128, k = 2048, S = 32768).  Both outputs are deterministic: each dkv row is the sum of its
 *   contributions in (query row, entry) order, with no atomic adds.  ds and p enter the head
 *   contraction of dkv as fp16 (ds times sm_scale), dq's contraction as a bf16 pair (16 significant
 *   bits); dout and q are converted bf16 -> fp16 for dkv (exact for |x| in [2^-14, 65504]).
 *   Supported: (D_qk, D_v) = (576, 512), 1 <= H <= 128, 1 <= k <= 2048; T = 0 with S > 0 zeroes dkv.
 */
size_t dsa_sparse_mla_bwd_workspace_size(int64_t T, int64_t S, int32_t H, int32_t k);
dsa_status_t dsa_sparse_mla_bwd(const uint16_t *q, const uint16_t *kv, const int32_t *indices, const float *lse,
                                const uint16_t *dout, int64_t T, int64_t S, int32_t H,
                                int32_t D_qk, int32_t D_v, int32_t k, int64_t q_start, float sm_scale, float *dq,
                                float *dkv, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Paged cache (summary page, section "Key claims": the released indexer-logit kernels include paged
 * versions).  Logical key s
 * of sequence b lives in block block_table[b][s / block_size], slot s % block_size, of the pools
 *   k8 [num_blocks][block_size][D_I] u8, k_scale [num_blocks][block_size] f32,
 *   kv [num_blocks][block_size][D_qk] bf16.
 * block_table [B][max_blocks_per_seq] i32; seq_lens [B] i32 (device; includes new tokens).
 * block_size must be a power of two (64 in the model deployment).
 * Precondition of the readers (prefill, decode): every block_table entry that covers a visible
 * position (s < q_start + T of the prefilled sequence; s < seq_lens[b] in decode) lies in
 * [0, num_blocks); entries past them are never read.  The table lives in device memory, so the
 * host cannot check it: an entry outside the pool is read as block 0 (no access leaves the
 * pools) and the scores and outputs of the affected rows are then unspecified.
 */
typedef struct {
  const uint8_t *k8;
  const float *k_scale;
  const uint16_t *kv;
  int64_t num_blocks;
  int32_t block_size;
  const int32_t *block_table;
  int64_t max_blocks_per_seq;
  const int32_t *seq_lens;
} dsa_paged_cache_t;

typedef struct {
  int32_t H_I, D_I, H, D_qk, D_v, topk;
  float sm_scale;
} dsa_dims_t;

/*
 * Fused prefill of sequence `seq`: T queries at positions q_start .. q_start + T - 1 over the
 * S = q_start + T keys already in the paged cache: indexer -> top-k -> sparse MLA, the same
 * kernels as the three standalone calls.  q8/q_scale/w/q as in the standalone calls,
 * out [T][H][D_v] bf16, out_f32 (optional), lse [T][H] (optional), indices_out [T][topk]
 * (optional; written when non-NULL).  Workspace: dsa_prefill_workspace_size() bytes, 256-byte
 * aligned; at (D_qk, D_v) = (576, 512) it includes the fp16 copy of the sequence's S latent rows
 * and the sparse MLA runs with fp16 staging (see dsa_sparse_mla_fwd; precondition |q|, |kv| <=
 * 65504).  T <= 1,048,576 per call, as dsa_indexer_logits.  Once the call's stream work has
 * completed, the first T * ld * 4 bytes of the workspace hold the index scores, fp32 [T][ld] with
 * ld = (S + 3) / 4 * 4 and entries s < n_t written (the scores the top-k selected from); the rest
 * of the workspace is private.
 */
size_t dsa_prefill_workspace_size(const dsa_dims_t *d, int64_t T, int64_t S);
dsa_status_t dsa_prefill_paged(const dsa_paged_cache_t *c, int32_t seq, const dsa_dims_t *d, int64_t T,
                               int64_t q_start, const uint8_t *q8, const float *q_scale, const float *w,
                               const uint16_t *q, uint16_t *out, float *out_f32, float *lse,
                               int32_t *indices_out, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * Fused decode: one new query per sequence b at position seq_lens[b] - 1 over its seq_lens[b]
 * keys (max_seq_len >= every seq_lens[b], used for grid and workspace sizing).
 * q8 [B][H_I][D_I], q_scale [B][H_I], w [B][H_I], q [B][H][D_qk], out [B][H][D_v],
 * out_f32 / lse / indices_out optional as above.  Sparse MLA is split over index chunks and the
 * partial results are re-reduced in fp32.  B <= 12288 (the per-sequence key-group prefix table of
 * the indexer sits in LDS; DSA_ERR_UNSUPPORTED above).
 * Workspace layout visible to the caller: once the call's stream work has completed, the first
 * B * ld * 4 bytes of the workspace hold the index scores, fp32 [B][ld] with
 * ld = (max_seq_len + 3) / 4 * 4 and entries s < seq_lens[b] of row b written (the scores the
 * top-k selected from; later entries are unspecified).  The rest of the workspace is private.
 */
size_t dsa_decode_workspace_size(const dsa_dims_t *d, int32_t B, int64_t max_seq_len);
dsa_status_t dsa_decode_paged(const dsa_paged_cache_t *c, int32_t B, int64_t max_seq_len,
                              const dsa_dims_t *d, const uint8_t *q8, const float *q_scale,
                              const float *w, const uint16_t *q, uint16_t *out, float *out_f32,
                              float *lse, int32_t *indices_out, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * FP8 quantization of indexer vectors (createthis gist page, indexer listing: the query and key
 * vectors are cast to FP8 E4M3 along the last dimension with one scale per vector).  Row r of
 * x (bf16 [rows][D]) becomes scales[r] = max_i |x[r][i]| / 448 (1 for an all-zero row) and
 * codes[r][i] = E4M3(clamp(x[r][i] / scales[r], -448, 448)): fp32 division, round to nearest
 * even, OCP E4M3 bit patterns.  codes u8 [rows][D], scales f32 [rows], device pointers, 16-byte
 * aligned.  D a multiple of 8 in [8, 512] (DSA_ERR_UNSUPPORTED otherwise).  For the indexer's
 * queries pass rows = T * H_I, D = D_I; the result is the q8 / q_scale of the calls above.
 */
dsa_status_t dsa_quantize_fp8_rows(const uint16_t *x, int64_t rows, int32_t D, uint8_t *codes, float *scales,
                                   hipStream_t stream);

/*
 * Power-of-two (UE8M0) variant of the quantizer (createthis gist page, indexer listing: the
 * cast helper's use_ue8m0 option): the scale of row r is 2^p_r, p_r the smallest integer with
 * 2^p_r >= max_i |x[r][i]| / 448 (fp32 division; 1 for an all-zero row), at least -127; exps[r] =
 * p_r + 127 (u8 [rows]); scales[r] = 2^p_r (f32 [rows], optional: NULL skips it); codes as above
 * with that scale.  Same shapes, alignment and D range as dsa_quantize_fp8_rows.
 */
dsa_status_t dsa_quantize_fp8_rows_ue8m0(const uint16_t *x, int64_t rows, int32_t D, uint8_t *codes,
                                         uint8_t *exps, float *scales, hipStream_t stream);

/*
 * Lightning-indexer scores with UE8M0 scales: the same scores as dsa_indexer_logits with
 * q_scale[t][j] = 2^(q_exp[t][j] - 127) and k_scale[s] = 2^(k_exp[s] - 127), the exponents
 * applied as the FP8 MFMA's own operand scales (gfx950 v_mfma_scale_f32_16x16x128_f8f6f4) rather
 * than in the epilogue.  q_exp u8 [T][H_I], k_exp u8 [S]; everything else as dsa_indexer_logits.
 */
dsa_status_t dsa_indexer_logits_ue8m0(const uint8_t *q8, const uint8_t *q_exp, const float *w, const uint8_t *k8,
                                      const uint8_t *k_exp, int64_t T, int64_t S, int32_t H_I, int32_t D_I,
                                      int64_t q_start, float *logits, int64_t ld_logits, hipStream_t stream);

/*
 * Paged append (summary page, section "Key claims": paged indexer caches).  Writes n new tokens
 * into the cache c: token i of sequence seq_ids[i] (0 <= seq_ids[i] < B, a row of
 * c->block_table) at position positions[i] gets, in physical row
 * block_table[seq][pos / block_size] * block_size + pos % block_size of the pools, the FP8 codes
 * and scale of its bf16 indexer key k[i] (D_I values, quantized as dsa_quantize_fp8_rows does)
 * and its bf16 latent row kv[i] (D_qk values, copied).  The pools behind c are written (the
 * const of the struct is the readers' view); seq_lens is not read or changed.  Tokens whose
 * sequence, position or block id falls outside the table or the pool are skipped.  Two tokens
 * mapped to the same slot race.  k bf16 [n][D_I], kv bf16 [n][D_qk], seq_ids / positions i32
 * [n], device pointers, 16-byte aligned; D_I as above, D_qk a positive multiple of 8.
 */
dsa_status_t dsa_append_paged(const dsa_paged_cache_t *c, int32_t B, const int32_t *seq_ids,
                              const int32_t *positions, int64_t n, int32_t D_I, int32_t D_qk, const uint16_t *k,
                              const uint16_t *kv, hipStream_t stream);

/*
 * Indexer training signal (summary page, section "Method", continued pre-training: in the dense
 * warm-up only the indexer is trained, against a KL-divergence target given by the main
 * attention).  Reading: for query row t and its visible keys s < n_t,
 *   p[t][s]  = (1/H) sum_h softmax_s(sm_scale * q[t][h][:] . kv[s][:])   (the main attention over
 *              every visible key, MQA: K = the whole latent row, averaged over the heads),
 *   pi[t][s] = softmax_s(logits[t][s]),
 *   loss[t]  = KL(p || pi) = sum_s p (log p - log pi)   (natural log; 0 log 0 = 0),
 *   dlogits[t][s] = pi[t][s] - p[t][s]   (the gradient of loss[t] with respect to logits[t][s]).
 *   q [T][H][D_qk] bf16, kv [S][D_qk] bf16, logits and dlogits [T][ld_logits] f32 (ld_logits >= S,
 *   a multiple of 4; dlogits may be logits itself, overwritten in place; entries s >= n_t are
 *   neither read nor written), loss [T] f32.  Scores must be finite.  Supported: 1 <= H <= 128,
 *   D_qk a multiple of 8 in [8, 576], S >= 1 when T > 0.
 */
dsa_status_t dsa_indexer_kl_loss(const uint16_t *q, const uint16_t *kv, int64_t T, int64_t S, int32_t H,
                                 int32_t D_qk, float sm_scale, int64_t q_start, const float *logits,
                                 int64_t ld_logits, float *dlogits, float *loss, hipStream_t stream);

/*
 * Sparse-stage indexer loss (summary page, "Method": once top-k is on, the indexer keeps its own
 * graph).  Reading: the loss of dsa_indexer_kl_loss restricted to the entries of each row's index
 * list.  For the valid entries i of indices[t] (0 <= idx < n_t; anything else is skipped; a key
 * listed twice counts once per entry, as in the sparse attention):
 *   p_i  = (1/H) sum_h exp(sm_scale * q[t][h][:] . kv[idx_i][:] - lse[t][h]),
 *   pi_i = softmax over the entries of logits[t][idx_i],   loss[t] = sum_i p_i (log p_i - log pi_i),
 *   dlogits[t][s] = sum_{i: idx_i = s} (pi_i - p_i) for s < n_t, 0 for visible keys not listed.
 *   lse [T][H] f32 is the natural-log normaliser of the sparse attention over the same lists (the
 *   lse output of dsa_sparse_mla_fwd); indices [T][k] i32; other arguments as dsa_indexer_kl_loss
 *   (dlogits may be logits itself).  A row without valid entries gets loss 0 and dlogits 0.
 *   Repeated keys are summed with atomic adds (their order is not fixed).  Supported: as
 *   dsa_indexer_kl_loss, 1 <= k <= 2048.
 */
dsa_status_t dsa_indexer_kl_loss_sparse(const uint16_t *q, const uint16_t *kv, const int32_t *indices, int32_t k,
                                        const float *lse, int64_t T, int64_t S, int32_t H, int32_t D_qk,
                                        float sm_scale, int64_t q_start, const float *logits, int64_t ld_logits,
                                        float *dlogits, float *loss, hipStream_t stream);

/*
 * Indexer backward (the same training stages): gradients of a loss through the scores of
 * dsa_indexer_logits given dlogits = dL/dlogits on the visible entries (s < n_t; others never
 * read).  Reading: the FP8 quantization is passed straight through, so the gradients are with
 * respect to the dequantized vectors q_I = q_scale dec(q8), k_I = k_scale dec(k8) and w, and
 * ReLU's derivative is 1 for a positive product and 0 otherwise; with z = q_I[t][j] . k_I[s]:
 *   dw[t][j] = sum_s dlogits[t][s] max(0, z),
 *   dq[t][j][:] = w[t][j] sum_{s: z > 0} dlogits[t][s] k_I[s][:],
 *   dk[s][:] = sum_{t, j: z > 0} dlogits[t][s] w[t][j] q_I[t][j][:].
 *   Inputs as dsa_indexer_logits (scales positive), dlogits [T][ld_dlogits] f32; outputs dq
 *   [T][H_I][D_I], dw [T][H_I], dk [S][D_I] f32 (every entry written).  The workspace (device,
 *   dsa_indexer_bwd_workspace_size() bytes) holds per-chunk partial key gradients; the result is
 *   deterministic.  Supported: H_I and D_I as dsa_indexer_logits, T and S both >= 1 (or both 0).
 */
size_t dsa_indexer_bwd_workspace_size(int64_t T, int64_t S, int32_t D_I);
dsa_status_t dsa_indexer_bwd(const uint8_t *q8, const float *q_scale, const float *w, const uint8_t *k8,
                             const float *k_scale, int64_t T, int64_t S, int32_t H_I, int32_t D_I, int64_t q_start,
                             const float *dlogits, int64_t ld_dlogits, float *dq, float *dw, float *dk,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Indexer backward of the sparse stage (summary page, "Method": the sparse-stage loss only sees
 * the selected keys, so dlogits vanishes off each row's index list).  Same gradients and
 * arguments as dsa_indexer_bwd, for a dlogits that is 0 at every visible key not in indices[t]
 * (as dsa_indexer_kl_loss_sparse writes it): dq and dw are summed over the valid entries of
 * indices [T][k] i32 only (0 <= idx < n_t; others skipped), dk as in dsa_indexer_bwd.  The
 * valid entries of a row must be distinct (top-k lists are): a key listed twice would be counted
 * twice in dq and dw.  Supported: as dsa_indexer_bwd, k >= 1.
 */
dsa_status_t dsa_indexer_bwd_listed(const uint8_t *q8, const float *q_scale, const float *w, const uint8_t *k8,
                                    const float *k_scale, int64_t T, int64_t S, int32_t H_I, int32_t D_I,
                                    int64_t q_start, const int32_t *indices, int32_t k, const float *dlogits,
                                    int64_t ld_dlogits, float *dq, float *dw, float *dk, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
