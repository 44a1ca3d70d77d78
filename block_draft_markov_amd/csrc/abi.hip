// C ABI of the draft step: argument validation (host side, before any
// launch), workspace layout and the launch sequence on the caller's stream.
// Declarations and the contract of every entry point: include/dflash_draft.h.

#include "../../include/dflash_draft.h"
#include "internal.hpp"

#include <cmath>

#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return DFLASH_OK;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(DFLASH_EHIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxRows = 1 << 20;
constexpr int64_t kMaxVocab = 1 << 26;
constexpr int64_t kMaxHidden = 1 << 16;
constexpr int64_t kMaxRank = 1 << 16;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int check_dims(const dflash_dims* d) {
    if (!d) return fail(DFLASH_EINVAL, "dims is NULL");
    if (d->num_requests < 0) return fail(DFLASH_EINVAL, "num_requests = %d < 0", d->num_requests);
    if (d->block_len < 1 || d->block_len > DFLASH_MAX_BLOCK_LEN)
        return fail(DFLASH_EINVAL, "block_len = %d outside [1, %d]", d->block_len, DFLASH_MAX_BLOCK_LEN);
    if (d->total_rows < 0 || d->total_rows > kMaxRows)
        return fail(DFLASH_EINVAL, "total_rows = %d outside [0, %lld]", d->total_rows, (long long)kMaxRows);
    if ((int64_t)d->total_rows > (int64_t)d->num_requests * d->block_len)
        return fail(DFLASH_EINVAL, "total_rows = %d exceeds num_requests * block_len = %lld", d->total_rows,
                    (long long)d->num_requests * d->block_len);
    if (d->hidden < 8 || d->hidden % 8 != 0 || d->hidden > kMaxHidden)
        return fail(DFLASH_EINVAL, "hidden = %d must be a multiple of 8 in [8, %lld]", d->hidden,
                    (long long)kMaxHidden);
    if (d->draft_vocab < 1 || d->draft_vocab > kMaxVocab)
        return fail(DFLASH_EINVAL, "draft_vocab = %d outside [1, %lld]", d->draft_vocab, (long long)kMaxVocab);
    if (d->target_vocab < d->draft_vocab || d->target_vocab > kMaxVocab)
        return fail(DFLASH_EINVAL, "target_vocab = %d must be in [draft_vocab = %d, %lld]", d->target_vocab,
                    d->draft_vocab, (long long)kMaxVocab);
    const int kmax = d->draft_vocab < DFLASH_MAX_TOP_K ? d->draft_vocab : DFLASH_MAX_TOP_K;
    if (d->top_k < 1 || d->top_k > kmax)
        return fail(DFLASH_EINVAL, "top_k = %d outside [1, min(64, draft_vocab) = %d]", d->top_k, kmax);
    if (d->rank < 1 || d->rank > kMaxRank)
        return fail(DFLASH_EINVAL, "rank = %d outside [1, %lld]", d->rank, (long long)kMaxRank);
    if (d->walk != DFLASH_WALK_VITERBI && d->walk != DFLASH_WALK_GREEDY)
        return fail(DFLASH_EINVAL, "walk = %d is neither DFLASH_WALK_VITERBI nor DFLASH_WALK_GREEDY", d->walk);
    if (d->options & ~DFLASH_OPT_FILTER_LOGITS)
        return fail(DFLASH_EINVAL, "options = %d has bits other than DFLASH_OPT_FILTER_LOGITS", d->options);
    if ((int64_t)dflash::topk_tiles_chunks(d->draft_vocab) * d->top_k > 2048)
        return fail(DFLASH_EUNSUPPORTED, "draft_vocab = %d is too large for top_k = %d", d->draft_vocab, d->top_k);
    return DFLASH_OK;
}

// rows of the packed blocks: uniform blocks need M = R * L exactly
int check_rows(const dflash_dims* d, const int32_t* row_offsets) {
    if (!row_offsets && (int64_t)d->total_rows != (int64_t)d->num_requests * d->block_len)
        return fail(DFLASH_EINVAL, "row_offsets is NULL but total_rows = %d != num_requests * block_len = %lld",
                    d->total_rows, (long long)d->num_requests * d->block_len);
    return DFLASH_OK;
}

// a required array: may be NULL only when it has no elements
int need(const void* p, int64_t count, const char* name) {
    if (count > 0 && !p) return fail(DFLASH_EINVAL, "%s is NULL", name);
    return DFLASH_OK;
}

struct Layout {
    int64_t ldz;
    int64_t ldt;      // tile maxima stride (0: none, the Top-K reads every logit)
    size_t logits, lse, part, tmax, cidx, ctok, unary, pair, dense, zs, tau, tmask, total;
    int nparts;
    int sample;       // vocabulary tiles sampled for the lm_head's logits filter (0: no filter)
};

Layout layout(const dflash_dims* d) {
    Layout l{};
    const int64_t M = d->total_rows, K = d->top_k;
    l.ldz = round_up(d->draft_vocab, 4);
    l.nparts = dflash::lmhead_partials(d->total_rows, d->draft_vocab);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = (size_t)round_up((int64_t)(off + bytes), 256);
        return at;
    };
    l.logits = take((size_t)(M * l.ldz) * sizeof(float));
    l.lse = take((size_t)M * sizeof(float));
    l.part = take((size_t)(M * l.nparts) * sizeof(float2));
    l.ldt = dflash::lmhead_has_tile_max(d->total_rows) ? (d->draft_vocab + 31) / 32 : 0;
    l.tmax = take((size_t)(M * l.ldt) * sizeof(float));
    l.cidx = take((size_t)(M * K) * sizeof(int32_t));
    l.ctok = take((size_t)(M * K) * sizeof(int64_t));
    l.unary = take((size_t)(M * K) * sizeof(float));
    l.pair = take((size_t)(M * K * K) * sizeof(float));
    l.dense = take((size_t)((int64_t)d->num_requests * d->block_len) * sizeof(uint64_t));
    l.sample = (d->options & DFLASH_OPT_FILTER_LOGITS) ? dflash::lmhead_sample_tiles(d->total_rows, d->draft_vocab)
                                                        : 0;
    l.zs = take((size_t)(M * 32 * l.sample) * sizeof(float));
    l.tau = take((size_t)(l.sample ? M : 0) * sizeof(float));
    l.tmask = take((size_t)(l.sample ? M * l.ldt : 0));
    l.total = off > 0 ? off : 256;
    return l;
}

int check_ws(const dflash_dims* d, const void* ws, size_t ws_bytes, Layout& l) {
    l = layout(d);
    if (!ws) return fail(DFLASH_EWORKSPACE, "workspace is NULL (%zu bytes needed)", l.total);
    if (ws_bytes < l.total)
        return fail(DFLASH_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes needed", ws_bytes,
                    l.total);
    if (!aligned(ws, 256)) return fail(DFLASH_EINVAL, "workspace is not 256-byte aligned");
    return DFLASH_OK;
}

template <class T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

constexpr int kSampled = 2;   // walk argument of whole_step: the sampled walk

// The whole step: validation, then the lm_head kernel, the Top-K from its tile
// maxima, the pair scores and the walk, in stream order.
int whole_step(const dflash_dims* d, const uint16_t* hidden, const uint16_t* lm_head, const int64_t* d2t,
               const float* tables, const float* gate_w, const int64_t* last_tok, const int32_t* row_offsets,
               int walk, const double* uniforms, float temperature, int64_t* tokens, float* scores, double* q,
               void* ws, size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_rows(d, row_offsets))) return rc;
    const int64_t M = d->total_rows, R = d->num_requests;
    if ((rc = need(hidden, M, "hidden")) || (rc = need(lm_head, 1, "lm_head")) ||
        (rc = need(tables, 1, "tables")) || (rc = need(last_tok, R, "last_tok")) ||
        (rc = need(tokens, M, "tokens")) || (rc = need(scores, R, "scores")))
        return rc;
    if (d->target_vocab > d->draft_vocab && !d2t)
        return fail(DFLASH_EINVAL, "target_vocab = %d > draft_vocab = %d needs d2t", d->target_vocab,
                    d->draft_vocab);
    if (gate_w && d2t)
        return fail(DFLASH_EUNSUPPORTED, "gate_w with d2t: gated (DFlash v2) drafts with a pruned vocabulary are "
                                         "not supported");
    if (!aligned(hidden, 16) || !aligned(lm_head, 16))
        return fail(DFLASH_EINVAL, "hidden and lm_head must be 16-byte aligned");
    Layout l;
    if ((rc = check_ws(d, ws, ws_bytes, l))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    float* logits = at<float>(ws, l.logits);
    float2* part = at<float2>(ws, l.part);
    float* tmax = at<float>(ws, l.tmax);
    // Logits filter (large batches): the exact logits of a sample of vocabulary tiles give
    // each row a bound tau at most its K-th largest logit; the lm_head kernel then writes only
    // the groups of four logits that reach tau (and a mask of them), and the Top-K reads only
    // those.  Every member of the top K is at least tau, so the slots are those of the
    // unfiltered logits.
    float* tau = nullptr;
    uint8_t* tmask = nullptr;
    if (l.sample > 0) {
        tau = at<float>(ws, l.tau);
        tmask = at<uint8_t>(ws, l.tmask);
        float* zs = at<float>(ws, l.zs);
        const int64_t ldzs = (int64_t)32 * l.sample;
        if ((e = dflash::launch_lmhead_sample(hidden, lm_head, d->total_rows, d->hidden, d->draft_vocab, l.sample,
                                              zs, ldzs, s)) != hipSuccess)
            return hip_fail(e, "lm_head sample launch");
        if ((e = dflash::launch_sample_tau(zs, ldzs, (int)ldzs, d->total_rows, d->top_k, tau, s)) != hipSuccess)
            return hip_fail(e, "sample bound launch");
    }
    // the lm_head kernel stores the tile maxima (there are some whenever there are rows)
    if ((e = dflash::launch_lmhead(hidden, lm_head, logits, l.ldz, part, tmax, l.ldt, d->total_rows, d->hidden,
                                   d->draft_vocab, s, tau, tmask)) != hipSuccess)
        return hip_fail(e, "lm_head launch");
    int32_t* cidx = at<int32_t>(ws, l.cidx);
    int64_t* ctok = at<int64_t>(ws, l.ctok);
    float* unary = at<float>(ws, l.unary);
    float* pair = at<float>(ws, l.pair);
    if ((e = dflash::launch_topk_tiles(logits, l.ldz, tmax, l.ldt, nullptr, part, l.nparts, d2t, d->total_rows,
                                       d->draft_vocab, d->top_k, cidx, ctok, unary, s, tmask, tau)) != hipSuccess)
        return hip_fail(e, "top-k launch");
    if ((e = dflash::launch_pair_scores(ctok, tables, gate_w, hidden, last_tok, row_offsets, d->num_requests,
                                        d->block_len, d->total_rows, d->hidden, d->target_vocab, d->top_k, d->rank,
                                        pair, s)) != hipSuccess)
        return hip_fail(e, "pair-score launch");
    if (walk == kSampled)
        e = dflash::launch_walk_sampled(ctok, unary, pair, row_offsets, d->num_requests, d->block_len, d->total_rows,
                                        d->top_k, uniforms, temperature, tokens, scores, nullptr, q, s);
    else
        e = dflash::launch_walk(ctok, unary, pair, row_offsets, d->num_requests, d->block_len, d->total_rows,
                                d->top_k, walk, tokens, scores, nullptr, s);
    if (e != hipSuccess)
        return hip_fail(e, "walk launch");
    return ok();
}

// The sampled walk's own arguments: a uniform per row, a finite positive temperature.
int check_sampling(const dflash_dims* d, const double* uniforms, float temperature) {
    if (!(temperature > 0.f) || !std::isfinite(temperature))
        return fail(DFLASH_EINVAL, "temperature = %g must be finite and positive", (double)temperature);
    return need(uniforms, d->total_rows, "uniforms");
}

// ---------------------------------------------------------------- static scratch
// The scratch of dflash_lattice_noalloc: the S lattice of the call, in a
// device array of the library (one copy per GPU, alive until the process
// ends), so that the call allocates nothing.  Host code never passes the
// array's name to a kernel: it takes the device address of the copy on the
// current GPU from hipGetSymbolAddress, once per device, and uses that.
constexpr size_t kScratchBytes = DFLASH_LATTICE_NOALLOC_MAX_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's copy of `scratch` (looked up on the first call per device).
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DFLASH_EINVAL, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(DFLASH_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DFLASH_OK;
}

// Host-side checks shared by dflash_lattice and dflash_lattice_noalloc.
int check_lattice(const dflash_dims* d, const int64_t* cand_tok, const float* unary, const float* tables,
                  const float* gate_w, const uint16_t* hidden, const int64_t* last_tok, const int32_t* row_offsets,
                  const int64_t* tokens, const float* scores) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_rows(d, row_offsets))) return rc;
    const int64_t M = d->total_rows, R = d->num_requests;
    if ((rc = need(cand_tok, M, "cand_tok")) || (rc = need(unary, M, "unary")) || (rc = need(tables, 1, "tables")) ||
        (rc = need(last_tok, R, "last_tok")) || (rc = need(tokens, M, "tokens")) || (rc = need(scores, R, "scores")))
        return rc;
    if (gate_w && (rc = need(hidden, M, "hidden (read by the gate)"))) return rc;
    return DFLASH_OK;
}

// Pair scores into `pair`, then the walk from them.
int launch_lattice(const dflash_dims* d, const int64_t* cand_tok, const float* unary, const float* tables,
                   const float* gate_w, const uint16_t* hidden, const int64_t* last_tok, const int32_t* row_offsets,
                   int64_t* tokens, float* scores, float* pair, hipStream_t s) {
    hipError_t e;
    if ((e = dflash::launch_pair_scores(cand_tok, tables, gate_w, hidden, last_tok, row_offsets, d->num_requests,
                                        d->block_len, d->total_rows, d->hidden, d->target_vocab, d->top_k, d->rank,
                                        pair, s)) != hipSuccess)
        return hip_fail(e, "pair-score launch");
    if ((e = dflash::launch_walk(cand_tok, unary, pair, row_offsets, d->num_requests, d->block_len, d->total_rows,
                                 d->top_k, d->walk, tokens, scores, nullptr, s)) != hipSuccess)
        return hip_fail(e, "walk launch");
    return DFLASH_OK;
}

}  // namespace

extern "C" {

size_t dflash_workspace_bytes(const dflash_dims* dims) {
    if (check_dims(dims) != DFLASH_OK) return 0;
    ok();
    return layout(dims).total;
}

int64_t dflash_logits_stride(int32_t draft_vocab) { return draft_vocab < 0 ? 0 : round_up(draft_vocab, 4); }

int dflash_draft_block(const dflash_dims* d, const uint16_t* hidden, const uint16_t* lm_head, const int64_t* d2t,
                       const float* tables, const float* gate_w, const int64_t* last_tok,
                       const int32_t* row_offsets, int64_t* tokens, float* scores, void* ws, size_t ws_bytes,
                       void* stream) {
    if (!d) return fail(DFLASH_EINVAL, "dims is NULL");
    return whole_step(d, hidden, lm_head, d2t, tables, gate_w, last_tok, row_offsets, d->walk, nullptr, 1.f, tokens,
                      scores, nullptr, ws, ws_bytes, stream);
}

int dflash_draft_block_sampled(const dflash_dims* d, const uint16_t* hidden, const uint16_t* lm_head,
                               const int64_t* d2t, const float* tables, const float* gate_w,
                               const int64_t* last_tok, const int32_t* row_offsets, const double* uniforms,
                               float temperature, int64_t* tokens, float* scores, double* q, void* ws,
                               size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_sampling(d, uniforms, temperature))) return rc;
    return whole_step(d, hidden, lm_head, d2t, tables, gate_w, last_tok, row_offsets, kSampled,
                      uniforms, temperature, tokens, scores, q, ws, ws_bytes, stream);
}

int dflash_draft_argmax(const dflash_dims* d, const uint16_t* hidden, const uint16_t* lm_head, const int64_t* d2t,
                        float out_scale, float soft_cap, int64_t* tokens, float* values, void* ws, size_t ws_bytes,
                        void* stream) {
    int rc;
    if ((rc = check_dims(d))) return rc;
    const int64_t M = d->total_rows;
    if ((rc = need(hidden, M, "hidden")) || (rc = need(lm_head, 1, "lm_head")) || (rc = need(tokens, M, "tokens")))
        return rc;
    if (!(out_scale > 0.f) || !std::isfinite(out_scale))
        return fail(DFLASH_EINVAL, "out_scale = %g must be finite and positive", (double)out_scale);
    if (!std::isfinite(soft_cap)) return fail(DFLASH_EINVAL, "soft_cap = %g must be finite", (double)soft_cap);
    if (d->target_vocab > d->draft_vocab && !d2t)
        return fail(DFLASH_EINVAL, "target_vocab = %d > draft_vocab = %d needs d2t", d->target_vocab,
                    d->draft_vocab);
    if (!aligned(hidden, 16) || !aligned(lm_head, 16))
        return fail(DFLASH_EINVAL, "hidden and lm_head must be 16-byte aligned");
    Layout l;
    if ((rc = check_ws(d, ws, ws_bytes, l))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    float* logits = at<float>(ws, l.logits);
    float* tmax = l.ldt ? at<float>(ws, l.tmax) : nullptr;
    if ((e = dflash::launch_lmhead(hidden, lm_head, logits, l.ldz, at<float2>(ws, l.part), tmax, l.ldt,
                                   d->total_rows, d->hidden, d->draft_vocab, s)) != hipSuccess)
        return hip_fail(e, "lm_head launch");
    if ((e = dflash::launch_argmax(logits, l.ldz, tmax, l.ldt, d2t, d->total_rows, d->draft_vocab, out_scale,
                                   soft_cap, tokens, values, s)) != hipSuccess)
        return hip_fail(e, "argmax launch");
    return ok();
}

int dflash_draft_dense(const dflash_dims* d, const uint16_t* hidden, const uint16_t* lm_head, const int64_t* d2t,
                       const float* tables, const int64_t* last_tok, const int32_t* row_offsets, float out_scale,
                       float soft_cap, int64_t* tokens, float* values, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_rows(d, row_offsets))) return rc;
    const int64_t M = d->total_rows, R = d->num_requests;
    if ((rc = need(hidden, M, "hidden")) || (rc = need(lm_head, 1, "lm_head")) || (rc = need(tables, 1, "tables")) ||
        (rc = need(last_tok, R, "last_tok")) || (rc = need(tokens, M, "tokens")))
        return rc;
    if (!(out_scale > 0.f) || !std::isfinite(out_scale))
        return fail(DFLASH_EINVAL, "out_scale = %g must be finite and positive", (double)out_scale);
    if (!std::isfinite(soft_cap)) return fail(DFLASH_EINVAL, "soft_cap = %g must be finite", (double)soft_cap);
    if (d->target_vocab > d->draft_vocab && !d2t)
        return fail(DFLASH_EINVAL, "target_vocab = %d > draft_vocab = %d needs d2t", d->target_vocab,
                    d->draft_vocab);
    if (!aligned(hidden, 16) || !aligned(lm_head, 16))
        return fail(DFLASH_EINVAL, "hidden and lm_head must be 16-byte aligned");
    Layout l;
    if ((rc = check_ws(d, ws, ws_bytes, l))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    float* logits = at<float>(ws, l.logits);
    if ((e = dflash::launch_lmhead(hidden, lm_head, logits, l.ldz, at<float2>(ws, l.part), nullptr, 0,
                                   d->total_rows, d->hidden, d->draft_vocab, s)) != hipSuccess)
        return hip_fail(e, "lm_head launch");
    if ((e = dflash::launch_dense_walk(logits, l.ldz, d2t, tables, last_tok, row_offsets, d->num_requests,
                                       d->block_len, d->total_rows, d->draft_vocab, d->target_vocab, d->rank,
                                       out_scale, soft_cap, at<uint64_t>(ws, l.dense), tokens, values, s)) !=
        hipSuccess)
        return hip_fail(e, "dense walk launch");
    return ok();
}

int dflash_lm_head(const dflash_dims* d, const uint16_t* hidden, const uint16_t* lm_head, float* logits,
                   int64_t ldz, float* lse, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_dims(d))) return rc;
    const int64_t M = d->total_rows;
    if ((rc = need(hidden, M, "hidden")) || (rc = need(lm_head, 1, "lm_head")) ||
        (rc = need(logits, M, "logits")))
        return rc;
    if (ldz < d->draft_vocab || ldz % 4 != 0)
        return fail(DFLASH_EINVAL, "ldz = %lld must be >= draft_vocab = %d and a multiple of 4", (long long)ldz,
                    d->draft_vocab);
    if (!aligned(hidden, 16) || !aligned(lm_head, 16) || !aligned(logits, 16))
        return fail(DFLASH_EINVAL, "hidden, lm_head and logits must be 16-byte aligned");
    Layout l;
    if ((rc = check_ws(d, ws, ws_bytes, l))) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    float2* part = at<float2>(ws, l.part);
    if ((e = dflash::launch_lmhead(hidden, lm_head, logits, ldz, part, nullptr, 0, d->total_rows, d->hidden, d->draft_vocab,
                                   s)) != hipSuccess)
        return hip_fail(e, "lm_head launch");
    if (lse && (e = dflash::launch_lse_combine(part, l.nparts, lse, d->total_rows, s)) != hipSuccess)
        return hip_fail(e, "lse launch");
    return ok();
}

int dflash_row_lse(const dflash_dims* d, const float* logits, int64_t ldz, float* lse, void* stream) {
    int rc;
    if ((rc = check_dims(d))) return rc;
    const int64_t M = d->total_rows;
    if ((rc = need(logits, M, "logits")) || (rc = need(lse, M, "lse"))) return rc;
    if (ldz < d->draft_vocab) return fail(DFLASH_EINVAL, "ldz = %lld < draft_vocab = %d", (long long)ldz,
                                          d->draft_vocab);
    hipError_t e = dflash::launch_row_lse(logits, ldz, lse, d->total_rows, d->draft_vocab,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "row lse launch");
    return ok();
}

int dflash_topk(const dflash_dims* d, const float* logits, int64_t ldz, const float* lse, const int64_t* d2t,
                int32_t* cand_idx, int64_t* cand_tok, float* unary, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_dims(d))) return rc;
    const int64_t M = d->total_rows, MK = M * d->top_k;
    if ((rc = need(logits, M, "logits")) || (rc = need(lse, M, "lse")) || (rc = need(cand_idx, MK, "cand_idx")) ||
        (rc = need(cand_tok, MK, "cand_tok")) || (rc = need(unary, MK, "unary")))
        return rc;
    if (ldz < d->draft_vocab || ldz % 4 != 0)
        return fail(DFLASH_EINVAL, "ldz = %lld must be >= draft_vocab = %d and a multiple of 4", (long long)ldz,
                    d->draft_vocab);
    if (!aligned(logits, 16)) return fail(DFLASH_EINVAL, "logits must be 16-byte aligned");
    if (d->target_vocab > d->draft_vocab && !d2t)
        return fail(DFLASH_EINVAL, "target_vocab = %d > draft_vocab = %d needs d2t", d->target_vocab,
                    d->draft_vocab);
    Layout l;
    if ((rc = check_ws(d, ws, ws_bytes, l))) return rc;
    // one streaming pass for the tile maxima, then the Top-K reads only the tiles they keep
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* tmax = at<float>(ws, l.tmax);
    hipError_t e = dflash::launch_tile_max(logits, ldz, d->total_rows, d->draft_vocab, tmax, l.ldt, s);
    if (e != hipSuccess) return hip_fail(e, "tile-maxima launch");
    if ((e = dflash::launch_topk_tiles(logits, ldz, tmax, l.ldt, lse, nullptr, 0, d2t, d->total_rows,
                                       d->draft_vocab, d->top_k, cand_idx, cand_tok, unary, s)) != hipSuccess)
        return hip_fail(e, "top-k launch");
    return ok();
}

int dflash_pair_scores(const dflash_dims* d, const int64_t* cand_tok, const float* tables, const float* gate_w,
                       const uint16_t* hidden, const int64_t* last_tok, const int32_t* row_offsets, float* pair,
                       void* stream) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_rows(d, row_offsets))) return rc;
    const int64_t M = d->total_rows, R = d->num_requests;
    if ((rc = need(cand_tok, M, "cand_tok")) || (rc = need(tables, 1, "tables")) ||
        (rc = need(last_tok, R, "last_tok")) || (rc = need(pair, M, "pair")))
        return rc;
    if (gate_w && (rc = need(hidden, M, "hidden (read by the gate)"))) return rc;
    hipError_t e = dflash::launch_pair_scores(cand_tok, tables, gate_w, hidden, last_tok, row_offsets,
                                              d->num_requests, d->block_len, d->total_rows, d->hidden,
                                              d->target_vocab, d->top_k, d->rank, pair,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pair-score launch");
    return ok();
}

int dflash_walk(const dflash_dims* d, const int64_t* cand_tok, const float* unary, const float* pair,
                const int32_t* row_offsets, int64_t* tokens, float* scores, int32_t* slots, void* stream) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_rows(d, row_offsets))) return rc;
    const int64_t M = d->total_rows, R = d->num_requests;
    if ((rc = need(cand_tok, M, "cand_tok")) || (rc = need(unary, M, "unary")) || (rc = need(pair, M, "pair")) ||
        (rc = need(tokens, M, "tokens")) || (rc = need(scores, R, "scores")))
        return rc;
    hipError_t e = dflash::launch_walk(cand_tok, unary, pair, row_offsets, d->num_requests, d->block_len,
                                       d->total_rows, d->top_k, d->walk, tokens, scores, slots,
                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "walk launch");
    return ok();
}

int dflash_lattice(const dflash_dims* d, const int64_t* cand_tok, const float* unary, const float* tables,
                   const float* gate_w, const uint16_t* hidden, const int64_t* last_tok, const int32_t* row_offsets,
                   int64_t* tokens, float* scores, void* ws, size_t ws_bytes, void* stream) {
    int rc;
    if ((rc = check_lattice(d, cand_tok, unary, tables, gate_w, hidden, last_tok, row_offsets, tokens, scores)))
        return rc;
    Layout l;
    if ((rc = check_ws(d, ws, ws_bytes, l))) return rc;
    if ((rc = launch_lattice(d, cand_tok, unary, tables, gate_w, hidden, last_tok, row_offsets, tokens, scores,
                             at<float>(ws, l.pair), static_cast<hipStream_t>(stream))))
        return rc;
    return ok();
}

int dflash_lattice_noalloc(const dflash_dims* d, const int64_t* cand_tok, const float* unary, const float* tables,
                           const float* gate_w, const uint16_t* hidden, const int64_t* last_tok,
                           const int32_t* row_offsets, int64_t* tokens, float* scores, void* stream) {
    int rc;
    if ((rc = check_lattice(d, cand_tok, unary, tables, gate_w, hidden, last_tok, row_offsets, tokens, scores)))
        return rc;
    const size_t need_bytes = (size_t)d->total_rows * (size_t)d->top_k * (size_t)d->top_k * sizeof(float);
    if (need_bytes > kScratchBytes)
        return fail(DFLASH_EINVAL, "total_rows * top_k^2 * 4 = %zu bytes exceeds the %zu-byte static scratch of "
                    "dflash_lattice_noalloc", need_bytes, kScratchBytes);
    if (d->num_requests == 0) return ok();   // nothing to launch
    void* sp = nullptr;
    if ((rc = scratch_address(&sp))) return rc;
    // every S entry the walk reads is written by the pair-score kernel first: nothing to clear
    if ((rc = launch_lattice(d, cand_tok, unary, tables, gate_w, hidden, last_tok, row_offsets, tokens, scores,
                             static_cast<float*>(sp), static_cast<hipStream_t>(stream))))
        return rc;
    return ok();
}

int dflash_walk_sampled(const dflash_dims* d, const int64_t* cand_tok, const float* unary, const float* pair,
                        const int32_t* row_offsets, const double* uniforms, float temperature, int64_t* tokens,
                        float* scores, int32_t* slots, double* q, void* stream) {
    int rc;
    if ((rc = check_dims(d)) || (rc = check_rows(d, row_offsets))) return rc;
    if ((rc = check_sampling(d, uniforms, temperature))) return rc;
    const int64_t M = d->total_rows, R = d->num_requests;
    if ((rc = need(cand_tok, M, "cand_tok")) || (rc = need(unary, M, "unary")) || (rc = need(pair, M, "pair")) ||
        (rc = need(tokens, M, "tokens")) || (rc = need(scores, R, "scores")))
        return rc;
    hipError_t e = dflash::launch_walk_sampled(cand_tok, unary, pair, row_offsets, d->num_requests, d->block_len,
                                               d->total_rows, d->top_k, uniforms, temperature, tokens, scores,
                                               slots, q, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sampled walk launch");
    return ok();
}

int dflash_check_d2t(const int64_t* d2t, int32_t Vd, int32_t Vt, int* is_injective) {
    if (!d2t) return fail(DFLASH_EINVAL, "d2t is NULL");
    if (!is_injective) return fail(DFLASH_EINVAL, "is_injective is NULL");
    if (Vd < 1 || Vt < Vd) return fail(DFLASH_EINVAL, "need 1 <= draft_vocab = %d <= target_vocab = %d", Vd, Vt);
    std::vector<uint8_t> seen((size_t)Vt, 0);
    int inj = 1;
    for (int32_t i = 0; i < Vd; ++i) {
        const int64_t t = (int64_t)i + d2t[i];
        if (t < 0 || t >= Vt)
            return fail(DFLASH_EINVAL, "d2t[%d] = %lld maps draft token %d to %lld, outside [0, %d)", i,
                        (long long)d2t[i], i, (long long)t, Vt);
        if (seen[(size_t)t]) inj = 0;
        seen[(size_t)t] = 1;
    }
    *is_injective = inj;
    return ok();
}

const char* dflash_last_error(void) { return g_err; }

}  // extern "C"
