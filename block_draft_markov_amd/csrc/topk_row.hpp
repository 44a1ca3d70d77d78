// The Top-K of one row (part 2 of the draft step) as a device function of a
// 256-thread workgroup: the K = min(64, V_d) best draft tokens of the row in
// slot order (logit descending, draft id ascending), the d2t remap of draft
// token i to target token i + d2t[i], and the unary score z - lse
// (optimum-intel page "Support MiniCPM-OCR-1.0-DSpark", What does this PR
// do?; the Markov head needs "the radix TopK" on the GPU per the page "Export
// DFlash v2 and DSpark drafts ...", What does this PR do?; ties ordered by
// index as in the TopP commit of the openvino.genai page).
//
// The top K of a row is read from the maxima of its 32-logit tiles: if tau is
// at most the K-th largest tile maximum, every member of the top K is >= tau and
// sits in a tile whose maximum reaches tau, so only those tiles are read.  The
// lm_head kernel stores the tile maxima as it writes the logits; for logits
// from elsewhere one streaming pass (tile_max in topk.hip) computes them.
// Within a chunk of a row (the exact path for rows with heavy ties), tau is the
// K-th largest of the 256 per-thread maxima: at least K keys of the chunk are
// >= tau, and only those survivors (about K + 10 for smooth rows) are ranked,
// each by counting the survivors that beat it, which yields the slot order
// directly.  When more than 256 keys survive, an exact radix select on 8-bit
// digits finds the K-th key instead, and equal keys are taken in id order.
// Sorted per-chunk lists are merged pairwise in LDS (each entry's merged
// position = its own index + the number of entries of the other list that beat
// it, by binary search).
// Entries are (key << 32 | ~id), so a larger entry is the better slot and
// every comparison is one 64-bit compare.
#pragma once

#include "common.hpp"

#include <math.h>

namespace dflash {

namespace {


constexpr int kThreads = 256;
constexpr int kFastCap = 256;   // survivors ranked directly
constexpr int kMaxTopK = 64;

__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int s = wsum[i];
        off += (i < w) ? s : 0;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return off + x - v;
}

// Slot-order the n unique entries of list[0..n) and write the first K to out
// (empty entries fill the rest when n < K).  list[n] must be readable and hold
// kEmptyEntry when n is odd (it is read in pairs and beats nothing).
__device__ __forceinline__ void rank_place(const uint64_t* list, int n, int K, uint64_t* out) {
    const ulonglong2* pairs = reinterpret_cast<const ulonglong2*>(list);
    const int np = (n + 1) >> 1;
    if (n <= kThreads / 2) {
        // two threads per entry, each counting the better entries in one half of the pairs
        const int i = threadIdx.x >> 1, h = threadIdx.x & 1;
        const uint64_t my = i < n ? list[i] : 0;
        const int half = (np + 1) >> 1;
        const int j0 = h * half, j1 = min(np, j0 + half);
        int rank = 0;
#pragma unroll 4
        for (int j = j0; j < j1; ++j) {
            const ulonglong2 e = pairs[j];
            rank += (e.x > my) ? 1 : 0;
            rank += (e.y > my) ? 1 : 0;
        }
        rank += __shfl_xor(rank, 1);
        if (i < n && h == 0 && rank < K) out[rank] = my;
        for (int k = n + threadIdx.x; k < K; k += kThreads) out[k] = kEmptyEntry;
        return;
    }
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const uint64_t my = list[i];
        int rank = 0;
#pragma unroll 4
        for (int j = 0; j < np; ++j) {
            const ulonglong2 e = pairs[j];
            rank += (e.x > my) ? 1 : 0;
            rank += (e.y > my) ? 1 : 0;
        }
        if (rank < K) out[rank] = my;
    }
    for (int i = n + threadIdx.x; i < K; i += kThreads) out[i] = kEmptyEntry;
}

// The q-th largest (1 <= q <= 64) of the 64 lanes' values, in every lane: the largest t with at
// least q lanes >= t, built bit by bit from the top (one ballot and one population count per
// bit, no exchange through LDS).  Every lane of the wave calls it.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t x, int q) {
    uint32_t t = 0;
#pragma unroll
    for (int b = 31; b >= 0; --b) {
        const uint32_t c = t | (1u << b);
        if (__popcll(__ballot(x >= c)) >= q) t = c;
    }
    return t;
}

struct ChunkShared {
    uint32_t wtau[4];
    __attribute__((aligned(16))) uint64_t cand[kFastCap + 2];
    uint32_t hist[256];
    int wsum[4];
    int s_digit, s_want;
};

// The K best entries of logits [cbase, cbase + 256 PT) of `row` (ids < V), slot
// ordered, into out[0..K) (global or LDS).  Called by all 256 threads; uses sh.
// mask (or NULL): bit (v / 4) % 8 of byte v / 32 tells whether logits v .. v + 3 (v % 4 == 0)
// were written; unwritten groups count as empty.
template <int PT>
__device__ __forceinline__ void chunk_select(const float* __restrict__ row, int cbase, int V, int K,
                                             uint64_t* out, ChunkShared& sh, const uint8_t* mask = nullptr) {
    const int tid = threadIdx.x;

    // ---- load PT logits per thread: element (j, q) has id cbase + j*1024 + 4*tid + q
    uint32_t key[PT];
#pragma unroll
    for (int j = 0; j < PT / 4; ++j) {
        const int v = cbase + j * (4 * kThreads) + 4 * tid;
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        bool put = v < V;
        if (put) {
            z = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + v));
            if (mask) put = (mask[v >> 5] >> ((v >> 2) & 7)) & 1;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) key[4 * j + q] = (put && v + q < V) ? float_to_key(z[q]) : 0u;
    }
    auto id_of = [&](int e) { return (uint32_t)(cbase + (e >> 2) * (4 * kThreads) + 4 * tid + (e & 3)); };

    // ---- tau: with q = ceil(K / 4), every wave has q lanes whose maximum is at
    // least the q-th largest lane maximum of that wave, so at least 4q >= K keys
    // of the chunk are >= the smallest of the four waves' q-th largest maxima.
    uint32_t mx = 0;
#pragma unroll
    for (int e = 0; e < PT; ++e) mx = max(mx, key[e]);
    const int q = (K + 3) >> 2;
    const uint32_t wq = wave_kth_largest(mx, q);
    if ((tid & 63) == 0) sh.wtau[tid >> 6] = wq;
    __syncthreads();
    const uint32_t tau = max(min(min(sh.wtau[0], sh.wtau[1]), min(sh.wtau[2], sh.wtau[3])), 1u);   // key 0: past the row

    int cnt = 0;
#pragma unroll
    for (int e = 0; e < PT; ++e) cnt += (key[e] >= tau) ? 1 : 0;
    int n;
    const int pos = block_excl_scan(cnt, sh.wsum, n);

    if (n <= kFastCap) {
        int p = pos;
#pragma unroll
        for (int e = 0; e < PT; ++e)
            if (key[e] >= tau && p < kFastCap) sh.cand[p++] = pack_entry(key[e], id_of(e));
        if (tid == 0) sh.cand[n] = kEmptyEntry;
        __syncthreads();
        rank_place(sh.cand, n, K, out);
        __syncthreads();
        return;
    }

    // ---- fallback: exact K-th key by radix select on 8-bit digits
    if (tid == 0) { sh.s_digit = 0; sh.s_want = 1; }
    uint32_t prefix = 0, pmask = 0;
    int want = K;
    for (int shift = 24; shift >= 0; shift -= 8) {
        sh.hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < PT; ++e)
            if (key[e] != 0u && (key[e] & pmask) == prefix) atomicAdd(&sh.hist[(key[e] >> shift) & 255u], 1u);
        __syncthreads();
        if (tid == 0) {
            int cum = 0;
            for (int d = 255; d >= 0; --d) {
                const int h = (int)sh.hist[d];
                if (cum + h >= want) { sh.s_digit = d; sh.s_want = want - cum; break; }
                cum += h;
            }
        }
        __syncthreads();
        prefix |= (uint32_t)sh.s_digit << shift;
        pmask |= 255u << shift;
        want = sh.s_want;
        __syncthreads();
    }
    const uint32_t T = prefix;   // the K-th largest key; `want` keys equal to T are taken
    int ngt_t = 0;
#pragma unroll
    for (int e = 0; e < PT; ++e) ngt_t += (key[e] > T) ? 1 : 0;
    int ngt;
    int p = block_excl_scan(ngt_t, sh.wsum, ngt);
#pragma unroll
    for (int e = 0; e < PT; ++e)
        if (key[e] > T && p < K) sh.cand[p++] = pack_entry(key[e], id_of(e));
    // equal keys in id order: id order is (j, thread, q)
    int taken_base = 0;
#pragma unroll
    for (int j = 0; j < PT / 4; ++j) {
        int neq = 0;
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) neq += (key[4 * j + q2] == T) ? 1 : 0;
        int tot;
        int ord = taken_base + block_excl_scan(neq, sh.wsum, tot);
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
            if (key[4 * j + q2] == T) {
                if (ord < want && ngt + ord < K) sh.cand[ngt + ord] = pack_entry(T, id_of(4 * j + q2));
                ++ord;
            }
        }
        taken_base += tot;
    }
    if (tid == 0) sh.cand[K] = kEmptyEntry;
    __syncthreads();
    rank_place(sh.cand, K, K, out);
    __syncthreads();
}

// Number of entries of the descending list y[0..n) that are > x (strict) or
// >= x (when `or_equal`).
__device__ __forceinline__ int count_better(const uint64_t* y, int n, uint64_t x, bool or_equal) {
    int lo = 0, hi = n;   // first index whose entry does not beat x
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const bool beats = or_equal ? (y[mid] >= x) : (y[mid] > x);
        if (beats) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// Merge nl slot-ordered lists of K entries held in LDS at a[0 .. nl K) (b is
// scratch of the same size) pairwise into one; returns the buffer holding it.
__device__ __forceinline__ uint64_t* merge_lists(uint64_t* a, uint64_t* b, int nl, int K) {
    const int tid = threadIdx.x;
    while (nl > 1) {
        const int pairs = nl >> 1;
        // one thread per entry of both lists of every pair
        for (int i = tid; i < pairs * 2 * K; i += kThreads) {
            const int pr = i / (2 * K), r = i % (2 * K);
            const uint64_t* x = a + (int64_t)(2 * pr) * K;
            const uint64_t* y = x + K;
            int dst;
            uint64_t e;
            if (r < K) { e = x[r]; dst = r + count_better(y, K, e, false); }
            else { e = y[r - K]; dst = (r - K) + count_better(x, K, e, true); }
            if (dst < K) b[(int64_t)pr * K + dst] = e;
        }
        if (nl & 1)
            for (int i = tid; i < K; i += kThreads) b[(int64_t)pairs * K + i] = a[(int64_t)(nl - 1) * K + i];
        __syncthreads();
        uint64_t* t = a; a = b; b = t;
        nl = pairs + (nl & 1);
    }
    return a;
}

// Slot k of row m from the final list: draft id, target id, unary score.
__device__ __forceinline__ void write_row(const uint64_t* list, int m, int K, int V, float lse,
                                          const int64_t* __restrict__ d2t, int32_t* __restrict__ cand_idx,
                                          int64_t* __restrict__ cand_tok, float* __restrict__ unary) {
    for (int k = threadIdx.x; k < K; k += kThreads) {
        const uint64_t e = list[k];
        uint32_t id = entry_id(e);
        id = min(id, (uint32_t)(V - 1));   // an empty entry cannot reach the top K when K <= V
        const float z = key_to_float(entry_key(e));
        const int64_t o = (int64_t)m * K + k;
        cand_idx[o] = (int32_t)id;
        cand_tok[o] = d2t ? (int64_t)id + d2t[id] : (int64_t)id;
        unary[o] = z - lse;
    }
}

// ---------------------------------------------------------------- from tile maxima
// When the lm_head kernel also stored the maximum of every 32-logit tile of
// every row, the top K of a row needs only a few of its tiles.  If tau is at
// most the K-th largest tile maximum, at least K logits are >= tau, so every
// member of the top K is >= tau and sits in a tile whose maximum is >= tau.
// tau comes from the per-thread maxima of the tile maxima as in chunk_select;
// the tiles it keeps (about K + 30 on smooth rows) are read, their logits
// >= tau ranked.  A row with more than kSelCap such tiles or kCandCap such
// logits (heavy ties) takes the exact path over all its logits instead.
constexpr int kSelCap = 1024;
constexpr int kCandCap = 512;
constexpr int kTileCap = 8192;   // tile-maxima keys kept in registers (32 per thread); longer rows re-read the rest
constexpr int kPartCap = 2048;   // lse partials loaded with the tile maxima (8 per thread); more are merged later

constexpr int kMaxListEntries = 2048;   // chunks * K of the exact path (checked on the host)

// Arguments of the Top-K of every row.  The lse of a row is lse_in[m] when lse_part is
// NULL, else merged from its nparts (max, sum exp) partials.
struct TopkRowArgs {
    const float* logits;
    int64_t ldz;
    const float* tmax;      // [M][ldt] tile maxima
    int64_t ldt;
    int tiles, V, K, nchunks;
    const float* lse_in;
    const float2* lse_part;
    int nparts;
    const int64_t* d2t;
    int32_t* cand_idx;
    int64_t* cand_tok;
    float* unary;
    const uint8_t* tmask;   // [M][ldt] groups of the tile written, or null (every logit written)
    const float* tau;       // [M] lower bound of the row's K-th largest logit, or null
};

__host__ __device__ inline int topk_chunks(int V) { return (V + kThreads * 64 - 1) / (kThreads * 64); }

inline TopkRowArgs topk_row_args(const float* logits, int64_t ldz, const float* tmax, int64_t ldt, const float* lse,
                                 const float2* lse_part, int nparts, const int64_t* d2t, int V, int K,
                                 int32_t* cand_idx, int64_t* cand_tok, float* unary,
                                 const uint8_t* tmask = nullptr, const float* tau = nullptr) {
    TopkRowArgs a;
    a.logits = logits; a.ldz = ldz; a.tmax = tmax; a.ldt = ldt;
    a.tiles = (V + 31) / 32; a.V = V; a.K = K; a.nchunks = topk_chunks(V);
    a.lse_in = lse; a.lse_part = lse_part; a.nparts = nparts; a.d2t = d2t;
    a.cand_idx = cand_idx; a.cand_tok = cand_tok; a.unary = unary;
    a.tmask = tmask; a.tau = tmask ? tau : nullptr;
    return a;
}

// LDS of the Top-K of one row.
struct TopkSmem {
    ChunkShared sh;
    int sel[kSelCap];
    __attribute__((aligned(16))) uint64_t cand[kCandCap + 2];
    uint64_t top[kMaxTopK];
    int s_nsel, s_ncand;
    float2 red[4];
    uint64_t lists[2 * kMaxListEntries];   // exact path: per-chunk lists and the merge scratch
};

// The Top-K of row m, by all 256 threads of the workgroup; writes cand_idx, cand_tok and
// unary of the row.
__device__ __forceinline__ void topk_row(const TopkRowArgs& a, int m, TopkSmem& s) {
    const float* __restrict__ logits = a.logits;
    const int64_t ldz = a.ldz;
    const float* __restrict__ tmax = a.tmax;
    const int64_t ldt = a.ldt;
    const int tiles = a.tiles, V = a.V, K = a.K, nchunks = a.nchunks;
    const float* __restrict__ lse_in = a.lse_in;
    const float2* __restrict__ lse_part = a.lse_part;
    const int nparts = a.nparts;
    const int64_t* __restrict__ d2t = a.d2t;
    int32_t* __restrict__ cand_idx = a.cand_idx;
    int64_t* __restrict__ cand_tok = a.cand_tok;
    float* __restrict__ unary = a.unary;
    const int tid = threadIdx.x;
    const float* row = logits + (int64_t)m * ldz;
    const float* trow = tmax + (int64_t)m * ldt;
    // ---- loads: the first kPartCap lse partials (or the caller's lse), then the first
    // kTileCap tile maxima, which are still in flight while the partials are merged
    constexpr int kTPT = kTileCap / kThreads;   // tile maxima per thread in the first round
    constexpr int kPPT = kPartCap / kThreads;   // lse partials per thread in the first round
    const float2* prow = lse_part ? lse_part + (int64_t)m * nparts : nullptr;
    // Every load below is issued by every lane (indices past the end are clamped and the
    // value replaced), so that the compiler can count the tile-maxima loads as issued after
    // the partials and wait for the partials alone.
    float2 pv[kPPT];
    if (prow) {
#pragma unroll
        for (int i = 0; i < kPPT; ++i) {
            const int idx = tid + kThreads * i;
            const float2 x = prow[idx < nparts ? idx : nparts - 1];
            pv[i] = idx < nparts ? x : make_float2(0.f, 0.f);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPPT; ++i) pv[i] = make_float2(0.f, 0.f);
    }
    const float lse_given = lse_part ? 0.f : lse_in[m];
    float tv[kTPT];
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
        const int t = tid + kThreads * i;
        const float x = trow[t < tiles ? t : tiles - 1];
        tv[i] = t < tiles ? x : 0.f;
    }
    // The lse is merged in two halves: each wave's (max, sum exp) into s.red[], then the four
    // waves after the next barrier.  The order of the merges is that of block_lse, so the
    // value is the same bit for bit.
    auto lse_wave = [&]() __attribute__((always_inline)) {
        if (!prow) return;
        float a = 0.f, sm = 0.f;
#pragma unroll
        for (int i = 0; i < kPPT; ++i) lse_merge(a, sm, pv[i].x, pv[i].y);
        for (int base = kPartCap; base < nparts; base += kPartCap) {
            float2 v[kPPT];
#pragma unroll
            for (int i = 0; i < kPPT; ++i) {
                const int idx = base + tid + kThreads * i;
                v[i] = idx < nparts ? prow[idx] : make_float2(0.f, 0.f);
            }
#pragma unroll
            for (int i = 0; i < kPPT; ++i) lse_merge(a, sm, v[i].x, v[i].y);
        }
        for (int o = 32; o > 0; o >>= 1) {
            const float m2 = __shfl_xor(a, o);
            const float s2 = __shfl_xor(sm, o);
            lse_merge(a, sm, m2, s2);
        }
        if ((tid & 63) == 0) s.red[tid >> 6] = make_float2(a, sm);
    };
    auto lse_final = [&]() __attribute__((always_inline)) {   // after a barrier that follows lse_wave
        if (!prow) return lse_given;
        float a = 0.f, sm = 0.f;
        for (int w = 0; w < 4; ++w) lse_merge(a, sm, s.red[w].x, s.red[w].y);
        return a + logf(sm);
    };

    lse_wave();

    // ---- tau from the tile maxima; their keys stay in registers
    uint32_t kv[kTPT];
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < kTPT; ++i) {
        const int t = tid + kThreads * i;
        kv[i] = t < tiles ? float_to_key(tv[i]) : 0u;   // 0 is below every tau
        mx = max(mx, kv[i]);
    }
    for (int t = kTileCap + tid; t < tiles; t += kThreads) mx = max(mx, float_to_key(trow[t]));
    const int q = (K + 3) >> 2;
    const uint32_t wq = wave_kth_largest(mx, q);
    if ((tid & 63) == 0) s.sh.wtau[tid >> 6] = wq;
    if (tid == 0) { s.s_nsel = 0; s.s_ncand = 0; }
    __syncthreads();
    uint32_t tau = max(min(min(s.sh.wtau[0], s.sh.wtau[1]), min(s.sh.wtau[2], s.sh.wtau[3])), 1u);
    // the lm_head's bound also has at least K logits at or above it (it is at most the K-th
    // largest), and every group of logits reaching it was written: the larger of the two
    // thresholds keeps the reads to written groups
    if (a.tau) tau = max(tau, float_to_key(a.tau[m]));
    const float lse = lse_final();
    const uint8_t* mrow = a.tmask ? a.tmask + (int64_t)m * ldt : nullptr;

    // ---- the tiles that may hold a member of the top K: a prefix count over the wave and
    // one LDS atomic per wave place each thread's tiles in s.sel[]
    {
        int c = 0;
#pragma unroll
        for (int i = 0; i < kTPT; ++i) c += kv[i] >= tau ? 1 : 0;
        const int lane = tid & 63;
        int x = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        int base = 0;
        if (lane == 63 && x > 0) base = atomicAdd(&s.s_nsel, x);
        base = __shfl(base, 63);
        int j = base + x - c;
#pragma unroll
        for (int i = 0; i < kTPT; ++i) {
            if (kv[i] >= tau) {
                if (j < kSelCap) s.sel[j] = tid + kThreads * i;
                ++j;
            }
        }
    }
    for (int t = kTileCap + tid; t < tiles; t += kThreads) {
        if (float_to_key(trow[t]) >= tau) {
            const int j = atomicAdd(&s.s_nsel, 1);
            if (j < kSelCap) s.sel[j] = t;
        }
    }
    __syncthreads();
    const int nsel = s.s_nsel;
    bool exact = nsel > kSelCap;
    if (!exact) {
        // ---- their logits >= tau (sixteen loads in flight per thread at a time: one round
        // for up to 128 tiles)
        float zv[16];
        uint32_t mk[16];   // the tile's mask (all groups written without one)
        auto load_round = [&](int base) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int e = base + tid + kThreads * i;
                const int v = e < nsel * 32 ? s.sel[e >> 5] * 32 + (e & 31) : V;
                zv[i] = v < V ? row[v] : 0.f;
                mk[i] = mrow && v < V ? mrow[v >> 5] : 0xFFu;
            }
        };
        auto scan_round = [&](int base) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int e = base + tid + kThreads * i;
                const int v = e < nsel * 32 ? s.sel[e >> 5] * 32 + (e & 31) : V;
                if (v < V && ((mk[i] >> ((v >> 2) & 7)) & 1u)) {
                    const uint32_t k = float_to_key(zv[i]);
                    if (k >= tau) {
                        const int c = atomicAdd(&s.s_ncand, 1);
                        if (c < kCandCap) s.cand[c] = pack_entry(k, (uint32_t)v);
                    }
                }
            }
        };
        for (int base = 0; base < nsel * 32; base += kThreads * 16) {
            load_round(base);
            scan_round(base);
        }
        __syncthreads();
        const int n = s.s_ncand;
        exact = n > kCandCap;
        if (!exact) {
            if (tid == 0) s.cand[n] = kEmptyEntry;
            __syncthreads();
            rank_place(s.cand, n, K, s.top);
            __syncthreads();
            write_row(s.top, m, K, V, lse, d2t, cand_idx, cand_tok, unary);
            return;
        }
    }
    // ---- exact path: every chunk of the row, then the merge, all in this workgroup
    for (int c = 0; c < nchunks; ++c)
        chunk_select<64>(row, c * (kThreads * 64), V, K, s.lists + (int64_t)c * K, s.sh, mrow);
    const uint64_t* fin = merge_lists(s.lists, s.lists + (int64_t)nchunks * K, nchunks, K);
    write_row(fin, m, K, V, lse, d2t, cand_idx, cand_tok, unary);
}

}  // namespace

}  // namespace dflash
