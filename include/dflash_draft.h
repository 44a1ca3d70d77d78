/*
 * dflash_draft.h — C ABI of the DFlash/DSpark draft step on MI355X (gfx950).
 *
 * The draft step turns the hidden states of the packed block rows of all
 * scheduled requests into drafted tokens, in four parts:
 *   1. lm_head projection to logits over the draft vocabulary
 *      (optimum-intel page "Support MiniCPM-OCR-1.0-DSpark", What does this
 *      PR do?: the draft applies its own lm_head over the draft vocabulary);
 *   2. Top-K per row, K = min(64, draft vocabulary), with the d2t remap of
 *      draft token i to target token i + d2t[i] (same page and section);
 *   3. the Markov-head candidate scorer over the K x K transitions between
 *      neighbouring positions, gated by the draft hidden states for DFlash v2
 *      (optimum-intel page "Export DFlash v2 and DSpark drafts ...", What does
 *      this PR do?; openvino.genai page "Add DSpark and DFlash v2 drafts ...",
 *      commit "DFlash-2 Markov head / BlockRowSource");
 *   4. a walk through that lattice for every request in one launch: the
 *      max-score path, or the greedy walk taking the best candidate after the
 *      token before (openvino.genai page, same commit).
 *
 * Scoring (the pages fix none; this is the definition the library computes):
 *   z_m[v]    = sum_i W[v,i] h_m[i]                (bf16 inputs, fp32 accumulation)
 *   lse_m     = log sum_v exp z_m[v]               (over the draft vocabulary)
 *   slots     = the K largest z_m, ordered by (z descending, draft id ascending)
 *   t_m[k]    = cand_m[k] + d2t[cand_m[k]]         (cand_m[k] when d2t is NULL)
 *   u_m[k]    = z_m[cand_m[k]] - lse_m
 *   g_m       = 1 / (1 + exp(-w . h_m)) when gate_w is given, else 1
 *   S_p[j][k] = g_m(p) * <A[t_{m(p-1)}[j]], B[t_{m(p)}[k]]>  for p >= 1,
 *   S_0[0][k] = g_m(0) * <A[last_tok], B[t_{m(0)}[k]]>
 *   Score(c)  = sum_p u_{m(p)}[c_p] + S_p[c_{p-1}][c_p]
 *   Viterbi: the max-Score path; at every max the lowest slot wins.
 *   Greedy:  c_p = lowest argmax_k u_{m(p)}[k] + S_p[c_{p-1}][k].
 *
 * Conventions shared by every entry point
 *   - Every pointer is caller-owned DEVICE memory unless stated otherwise.
 *     The library allocates nothing, keeps no state between calls and is
 *     re-entrant; all work is enqueued on `stream` (a hipStream_t; NULL is
 *     the null stream) and outputs are valid once the caller has
 *     synchronised with that stream.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Inputs must not alias outputs or the workspace.
 *   - Return value: DFLASH_OK (0) or a negative DFLASH_E* code.  On any error
 *     nothing is launched and no output is written; dflash_last_error()
 *     names the offending argument.  Argument checks are host-side and
 *     happen before any launch.
 *   - Device-data preconditions that the host cannot see (token ids in
 *     range, 0 <= i + d2t[i] < V_t, row_offsets well formed) are the caller's;
 *     dflash_check_d2t() checks d2t once on the host.  Kernels clamp every
 *     index they read so that a broken precondition gives wrong tokens, never
 *     an out-of-bounds access.
 *   - Inputs must be finite; NaN or Inf logits give unspecified tokens.
 */
#ifndef DFLASH_DRAFT_H
#define DFLASH_DRAFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_OK            0
#define DFLASH_EINVAL       -1  /* a bad size, a NULL required pointer, a bad mode */
#define DFLASH_EUNSUPPORTED -2  /* a legal but unsupported combination */
#define DFLASH_EWORKSPACE   -3  /* workspace NULL or smaller than dflash_workspace_bytes() */
#define DFLASH_EHIP         -4  /* the HIP runtime reported an error (message in dflash_last_error) */

#define DFLASH_WALK_VITERBI  0  /* max-score path over all K^L paths */
#define DFLASH_WALK_GREEDY   1  /* best candidate after the token before, position by position */

#define DFLASH_MAX_TOP_K     64
/* A block is at most num_assistant_tokens rows, which GenerationConfig
 * validation caps at 100 (openvino.genai page, the docs commit on the
 * num_assistant_tokens limit). */
#define DFLASH_MAX_BLOCK_LEN 100

/* Sizes of one call.  M = total_rows packed block rows; without row_offsets
 * every request owns block_len consecutive rows and total_rows must equal
 * num_requests * block_len; with row_offsets request r owns rows
 * row_offsets[r] .. row_offsets[r+1]-1, each at most block_len of them. */
typedef struct dflash_dims {
    int32_t num_requests;  /* R >= 0 */
    int32_t block_len;     /* L in [1, 100]: rows per request (the maximum with row_offsets) */
    int32_t total_rows;    /* M >= 0 */
    int32_t hidden;        /* H >= 8, a multiple of 8 */
    int32_t draft_vocab;   /* V_d >= 1 */
    int32_t target_vocab;  /* V_t >= V_d; V_t > V_d needs d2t */
    int32_t top_k;         /* K in [1, min(64, V_d)] */
    int32_t rank;          /* r >= 1, table rank */
    int32_t walk;          /* DFLASH_WALK_VITERBI or DFLASH_WALK_GREEDY */
    int32_t options;       /* 0, or DFLASH_OPT_FILTER_LOGITS */
} dflash_dims;

/* options: the whole-step calls (dflash_draft_block, dflash_draft_block_sampled) with more
 * than 64 rows and at least 512 vocabulary tiles of 32 logits never write the fp32 logits
 * that cannot reach the top K: the exact logits of 128 sampled tiles give each row a bound
 * (their K-th largest, at most the row's K-th largest logit), the lm_head kernel writes only
 * the groups of four logits whose maximum reaches it, with a mask of them, and the Top-K reads
 * only those.  The slots, tokens and scores are those of the unfiltered step, bit for bit.
 * Off by default: on MI355X the sample costs more than the writes it saves at the Qwen3-4B
 * and 27B shapes.  Other entry points ignore it. */
#define DFLASH_OPT_FILTER_LOGITS 1

/* Bytes of workspace every entry point below needs for these dims (the same
 * number for all of them), or 0 with dflash_last_error() set if the dims are
 * invalid.  The workspace must be device memory aligned to 256 bytes. */
size_t dflash_workspace_bytes(const dflash_dims* dims);

/* Row stride, in floats, of the logits buffers the stage entry points take:
 * draft_vocab rounded up to a multiple of 4 (16-byte aligned rows). */
int64_t dflash_logits_stride(int32_t draft_vocab);

/* The whole draft step (parts 1-4) in one call.
 *   hidden      bf16 [M][H] row-major: draft hidden states of the packed block rows
 *   lm_head     bf16 [V_d][H] row-major (nn.Linear layout): the draft lm_head
 *   d2t         int64 [V_d] or NULL: target id of draft token i is i + d2t[i]
 *   tables      fp32 [2][V_t][r]: tables[0] = A (indexed by the previous token),
 *               tables[1] = B (indexed by the candidate token)
 *   gate_w      fp32 [H] or NULL: gated (DFlash v2) transitions when given
 *   last_tok    int64 [R]: the last accepted target token of every request
 *   row_offsets int32 [R+1] or NULL (uniform blocks of block_len rows)
 *   tokens      out int64 [M]: drafted target token of every row
 *   scores      out fp32 [R]: Score of the chosen path (0 for a request without rows)
 *   workspace   device scratch of dflash_workspace_bytes(dims) bytes
 * gate_w together with d2t returns DFLASH_EUNSUPPORTED: DFlash v2 drafts with a
 * pruned vocabulary are rejected (optimum-intel page "Support
 * MiniCPM-OCR-1.0-DSpark", What does this PR do?). */
int dflash_draft_block(const dflash_dims* dims,
                       const uint16_t* hidden, const uint16_t* lm_head,
                       const int64_t* d2t, const float* tables, const float* gate_w,
                       const int64_t* last_tok, const int32_t* row_offsets,
                       int64_t* tokens, float* scores,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Part 1 (optimum-intel page "Support MiniCPM-OCR-1.0-DSpark", What does this
 * PR do?: the draft applies its own lm_head and outputs logits over the draft
 * vocabulary): logits[m][v] (fp32, row stride ldz >= V_d, ldz % 4 == 0) of
 * every row and lse[m] (fp32 [M], or NULL to skip it), from bf16 hidden [M][H]
 * and lm_head [V_d][H].  The per-row (max, sum exp) partials stay in the
 * workspace; logits and lse are caller-owned outputs. */
int dflash_lm_head(const dflash_dims* dims, const uint16_t* hidden, const uint16_t* lm_head,
                   float* logits, int64_t ldz, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream);

/* The unary's normaliser (the log-softmax over the draft vocabulary, the
 * reading of optimum-intel page "Support MiniCPM-OCR-1.0-DSpark", Tests: the
 * reference scores over the draft vocabulary): lse[m] = log sum_v exp
 * logits[m][v] over the first V_d entries of every row (row stride ldz >= V_d),
 * for logits that did not come from dflash_lm_head.  No workspace. */
int dflash_row_lse(const dflash_dims* dims, const float* logits, int64_t ldz, float* lse,
                   void* stream);

/* Part 2 (optimum-intel page "Export DFlash v2 and DSpark drafts ...", What
 * does this PR do?: the radix TopK of the head; optimum-intel page "Support
 * MiniCPM-OCR-1.0-DSpark", What does this PR do?: K = min(64, draft vocabulary)
 * and draft token i -> target token i + d2t[i]; ties ordered by index as in the
 * TopP commit of the openvino.genai page): the K slots of every row in slot
 * order (logit descending, draft id ascending).
 *   logits fp32 [M][ldz] (ldz >= V_d, ldz % 4 == 0, 16-byte aligned),
 *   lse fp32 [M], d2t int64 [V_d] or NULL (needed when V_t > V_d)
 *   cand_idx out int32 [M][K] draft ids; cand_tok out int64 [M][K] target ids;
 *   unary out fp32 [M][K] = z - lse. */
int dflash_topk(const dflash_dims* dims, const float* logits, int64_t ldz, const float* lse,
                const int64_t* d2t, int32_t* cand_idx, int64_t* cand_tok, float* unary,
                void* workspace, size_t workspace_bytes, void* stream);

/* Part 3 (optimum-intel page "Export DFlash v2 and DSpark drafts ...", What
 * does this PR do?: the Top-K lattice, transitions gated by the draft hidden
 * states for DFlash v2; openvino.genai page "Add DSpark and DFlash v2 drafts
 * ...", commit "DFlash-2 Markov head / BlockRowSource": one scorer run over
 * the packed rows of all requests): transition scores of every row, out fp32
 * pair [M][K][K] (caller-owned, no workspace):
 * pair[m(p)][j][k] = S_p[j][k] for p >= 1; for p = 0 row j = 0 holds S_0[0][k]
 * and rows j >= 1 are written as 0.
 *   cand_tok int64 [M][K], tables fp32 [2][V_t][r], gate_w fp32 [H] or NULL,
 *   hidden bf16 [M][H] (read only when gate_w is given), last_tok int64 [R],
 *   row_offsets int32 [R+1] or NULL. */
int dflash_pair_scores(const dflash_dims* dims, const int64_t* cand_tok, const float* tables,
                       const float* gate_w, const uint16_t* hidden, const int64_t* last_tok,
                       const int32_t* row_offsets, float* pair, void* stream);

/* Part 4 (openvino.genai page "Add DSpark and DFlash v2 drafts ...", commit
 * "DFlash-2 Markov head / BlockRowSource": the greedy walk takes the best
 * candidate after the token before; the max-score walk is its Viterbi form):
 * the walk of every request over unary fp32 [M][K] and pair fp32 [M][K][K] (as
 * written by dflash_pair_scores), one launch for all requests, no workspace.
 *   tokens out int64 [M] = cand_tok[m][c_p]; scores out fp32 [R];
 *   slots out int32 [M] (the chosen slot c_p of every row) or NULL. */
int dflash_walk(const dflash_dims* dims, const int64_t* cand_tok, const float* unary,
                const float* pair, const int32_t* row_offsets,
                int64_t* tokens, float* scores, int32_t* slots, void* stream);

/* Parts 3 and 4 in one call: the candidate scorer over the packed block rows
 * of all requests, then the walk (openvino.genai page "Add DSpark and DFlash
 * v2 drafts ...", commit "DFlash-2 Markov head / BlockRowSource": the Top-K
 * scorer runs once over the packed rows of every scheduled request and the
 * walk then takes the candidates request by request).
 *   cand_tok    int64 [M][K] target ids of the slots (slot order, as dflash_topk writes)
 *   unary       fp32 [M][K] unary score of every slot
 *   tables      fp32 [2][V_t][r]; gate_w fp32 [H] or NULL; hidden bf16 [M][H]
 *               (read only when gate_w is given, may be NULL otherwise)
 *   last_tok    int64 [R]; row_offsets int32 [R+1] or NULL
 *   tokens      out int64 [M] = cand_tok[m][c_p]; scores out fp32 [R] (0 for a
 *               request without rows)
 *   workspace   dflash_workspace_bytes(dims) bytes, 256-byte aligned; holds S
 * dims->draft_vocab only bounds top_k here.  Token ids must lie in [0, V_t)
 * (the kernels clamp them).  Same results as dflash_pair_scores followed by
 * dflash_walk, bit for bit. */
int dflash_lattice(const dflash_dims* dims, const int64_t* cand_tok, const float* unary, const float* tables,
                   const float* gate_w, const uint16_t* hidden, const int64_t* last_tok,
                   const int32_t* row_offsets, int64_t* tokens, float* scores,
                   void* workspace, size_t workspace_bytes, void* stream);

/* dflash_lattice for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, kernels and results as dflash_lattice, without the
 * workspace: S lives in a static device array of the library,
 * DFLASH_LATTICE_NOALLOC_MAX_BYTES bytes per GPU, held until the process ends.
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 *   Limit: total_rows * top_k^2 * 4 <= DFLASH_LATTICE_NOALLOC_MAX_BYTES
 *          (1024 rows at K = 64); larger calls return DFLASH_EINVAL.
 *   The array of a GPU is shared by every call on it and keeps the last
 *   call's contents (every entry a call reads is written by that call first):
 *   calls that overlap on one GPU (other streams, other threads) race and must
 *   be serialised by the caller.  The GPU is the device current on the calling
 *   thread; the stream and every buffer must belong to it. */
#define DFLASH_LATTICE_NOALLOC_MAX_BYTES (16u << 20)
int dflash_lattice_noalloc(const dflash_dims* dims, const int64_t* cand_tok, const float* unary,
                           const float* tables, const float* gate_w, const uint16_t* hidden,
                           const int64_t* last_tok, const int32_t* row_offsets,
                           int64_t* tokens, float* scores, void* stream);

/* Sampled drafting (openvino.genai page "Add DSpark and DFlash v2 drafts and
 * sampled drafting ...", commit "DFlash-2 Markov head / BlockRowSource": a
 * sampled request walks the lattice with the request's draft RNG; the
 * sampled-drafting commits of the same page: the weights are float exps, their
 * running and total sums doubles, the uniform a double, and the proposal of
 * every drawn candidate is recorded for the target's rejection sampling).
 * The caller's RNG supplies the uniforms, so a draw is a function of them.
 * For request r, position p (row m), c_{-1} selecting row 0 of S_0:
 *   x_k = fp32(fp32(u_m[k] + S_p[c_{p-1}][k]) / temperature)
 *   w_k = fp32(exp(x_k - max_j x_j))        (rounded from a double exp)
 *   W_k = w_0 + ... + w_k in double, in slot order; total = W_{K-1}
 *   c_p = the smallest k with uniforms[m] * total < W_k (K - 1 if none)
 *   q[m][k] = w_k / total (double)
 *   uniforms  double [M] in [0, 1), one per row
 *   temperature finite and > 0 (DFLASH_EINVAL otherwise)
 *   q         out double [M][K] or NULL: the proposal each slot was drawn from
 *   scores    out fp32 [R]: Score(c) of the drawn path (as dflash_draft_block)
 * Everything else as dflash_draft_block; dims->walk must be valid and is not
 * used. */
int dflash_draft_block_sampled(const dflash_dims* dims,
                               const uint16_t* hidden, const uint16_t* lm_head,
                               const int64_t* d2t, const float* tables, const float* gate_w,
                               const int64_t* last_tok, const int32_t* row_offsets,
                               const double* uniforms, float temperature,
                               int64_t* tokens, float* scores, double* q,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Part 4 sampled: the walk above from given candidates, unary and S (the
 * layouts of dflash_walk); slots out int32 [M] or NULL. */
int dflash_walk_sampled(const dflash_dims* dims, const int64_t* cand_tok, const float* unary,
                        const float* pair, const int32_t* row_offsets,
                        const double* uniforms, float temperature,
                        int64_t* tokens, float* scores, int32_t* slots, double* q, void* stream);

/* Head-less draft step (openvino.genai page, commit "DFlash-2 Markov head /
 * BlockRowSource": without a Markov head the selector scales and soft caps
 * the backbone rows, and a greedy request takes the best token of every row).
 * For every row m of hidden bf16 [M][H]:
 *   z'_m[v] = soft_cap * tanh(out_scale * z_m[v] / soft_cap)   when soft_cap > 0,
 *           = out_scale * z_m[v]                               otherwise,
 *   with z_m = W h_m as in dflash_draft_block;
 *   tokens out int64 [M] = t(i_m), i_m = the lowest draft id maximizing z'_m,
 *   t(i) = i + d2t[i] (i when d2t is NULL);
 *   values out fp32 [M] = z'_m[i_m], or NULL to skip.
 * dims: total_rows, hidden, draft_vocab and target_vocab as for
 * dflash_draft_block (the other fields must be valid and are not used).
 * out_scale must be finite and > 0 (DFLASH_EINVAL otherwise); soft_cap must
 * be finite.  Workspace: dflash_workspace_bytes(dims) bytes, 256-byte aligned.
 * The maximum is taken in fp32 on the kernel's z' values. */
int dflash_draft_argmax(const dflash_dims* dims, const uint16_t* hidden, const uint16_t* lm_head,
                        const int64_t* d2t, float out_scale, float soft_cap, int64_t* tokens,
                        float* values, void* workspace, size_t workspace_bytes, void* stream);

/* Dense Markov walk (openvino.genai page "Add DSpark and DFlash v2 drafts ...",
 * Description: with markov_head_top_k = 0 the head, DSpark only, corrects
 * every drafted position, one inference per position; commit "DFlash-2 Markov
 * head / BlockRowSource": the dense step biases the scaled rows by the token
 * drafted before and a greedy request takes the best biased token).  For
 * request r with rows m(0) .. m(n-1), s_0 = last_tok[r]:
 *   x_p[v] = z'_{m(p)}[v] + <A[s_p], B[t(v)]>   over all draft ids v,
 *   c_p    = the lowest draft id maximizing x_p,   s_{p+1} = t(c_p),
 * z' the scaled, soft-capped rows of dflash_draft_argmax, t and the tables
 * fp32 [2][V_t][r] as in dflash_draft_block (no gate).
 *   tokens out int64 [M] = t(c_p); values out fp32 [M] = x_p[c_p], or NULL.
 * dims as for dflash_draft_block (top_k and walk must be valid and are not
 * used); row_offsets int32 [R+1] or NULL; out_scale finite and > 0,
 * soft_cap finite (DFLASH_EINVAL otherwise).  Workspace:
 * dflash_workspace_bytes(dims) bytes, 256-byte aligned.  Products and sums in
 * fp32; the maximum is taken in fp32 on the kernel's x values.  One launch per
 * position follows the lm_head launch on `stream`. */
int dflash_draft_dense(const dflash_dims* dims, const uint16_t* hidden, const uint16_t* lm_head,
                       const int64_t* d2t, const float* tables, const int64_t* last_tok,
                       const int32_t* row_offsets, float out_scale, float soft_cap,
                       int64_t* tokens, float* values, void* workspace, size_t workspace_bytes,
                       void* stream);

/* HOST memory: checks once, at set-up, that every i + d2t[i] lies in
 * [0, V_t) (returns DFLASH_EINVAL naming the first bad i otherwise) and
 * writes 1 to *is_injective when no two draft ids share a target id, else 0
 * (openvino.genai page, d2t commit: the size is checked per call, injectivity
 * once; greedy drafting accepts any mapping). */
int dflash_check_d2t(const int64_t* d2t_host, int32_t draft_vocab, int32_t target_vocab,
                     int* is_injective);

/* Message of the last error on the calling thread ("" after success). */
const char* dflash_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_DRAFT_H */
