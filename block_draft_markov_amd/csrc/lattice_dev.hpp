// Parts 3 and 4 of the draft step as device functions of one workgroup, run by
// the kernels of lattice.hip: the Markov-head candidate scorer over the packed
// Top-K lattice and the walk through it.
//
// Scorer (optimum-intel page "Export DFlash v2 and DSpark drafts ...", What
// does this PR do?: the Top-K lattice of the DSpark head, with transitions
// gated by the draft hidden states for DFlash v2; openvino.genai page "Add
// DSpark and DFlash v2 drafts ...", commit "DFlash-2 Markov head /
// BlockRowSource": one run over the packed block rows of all requests):
//   S_p[j][k] = g_p * <A[t_{p-1}[j]], B[t_p[k]]>,  S_0[0][k] = g_0 * <A[last], B[t_0[k]]>,
//   g_p = sigmoid(w . h_p) when gated, else 1.
// One workgroup per (position, request).  The K rows of A and of B it needs
// are gathered 256 rank elements at a time, in four phases with two in flight,
// into LDS rows of 260 floats (the 32 rows a wave reads fall in distinct
// banks); eight waves compute S with fp32 MFMAs, two per 32 x 32 quadrant, each
// over one half of the rank, starting as soon as their phases have landed.
//
// Walk (same commit: the greedy walk takes the best candidate after the token
// before; the max-score walk is its Viterbi form): one 256-thread workgroup per
// request.  Viterbi: thread (k, q) takes the best delta(j) + S[j][k] over j in
// its quarter q of the slots (ascending, strict >), and the quarters are
// combined in order, so the lowest j wins a tie; a block of at most 16
// positions keeps S, u and the back-pointers in registers, a longer one stages
// four positions of S and u at a time in two LDS buffers.  Greedy: one wave, an
// argmax per position (DPP max reduction, lowest lane of a ballot).  Sampled
// (same commit: a sampled request walks the lattice with its draft RNG; the
// sampled-drafting commits: float weights, double sums, a double uniform, the
// proposal recorded for rejection sampling): one wave; per position the row
// after the slot drawn before, one caller-supplied uniform per row.
#pragma once

#include "common.hpp"
#include "lds_dma.hpp"
#include "../../include/dflash_draft.h"

#include <math.h>

namespace dflash {

namespace {

constexpr int kLatThreads = 256;    // threads of a walk workgroup: four waves
constexpr int kPairThreads = 512;   // threads of a scorer workgroup: eight waves
constexpr int kGateRounds = 2;      // gate: rounds of 8 elements per thread whose loads are all issued first
constexpr int kRankSlice = 256;     // rank elements staged per round
constexpr int kPitch = kRankSlice + 4;   // LDS row pitch (floats): 16 consecutive rows hit distinct banks
constexpr int kWalkSampled = 2;     // the sampled walk (its own entry points; not a dims.walk value)
constexpr int kWalkChunk = 4;       // positions of S and u per LDS buffer; two buffers
constexpr int kRegPositions = 16;   // Viterbi blocks of at most this many positions keep S in registers

// Rows of request req: [a, a + n), n at most L (uniform blocks of L rows without offsets).
__device__ __forceinline__ void row_range(const int32_t* row_offsets, int req, int L, int M, int& a, int& n) {
    if (row_offsets) {
        int lo = row_offsets[req], hi = row_offsets[req + 1];
        lo = min(max(lo, 0), M);
        hi = min(max(hi, lo), M);
        a = lo;
        n = min(hi - lo, L);
    } else {
        a = req * L;
        n = L;
    }
}

__device__ __forceinline__ int64_t clamp_tok(int64_t t, int Vt) {
    return t < 0 ? 0 : (t >= Vt ? (int64_t)Vt - 1 : t);
}

struct PairArgs {
    const int64_t* cand_tok;     // [M][K] target ids of the slots
    const float* tables;         // [2][Vt][r]
    const float* gate_w;         // [H] or null
    const uint16_t* hidden;      // [M][H] bf16 (read when gated)
    const int64_t* last_tok;     // [R]
    const int32_t* row_offsets;  // [R+1] or null
    int L, M, H, Vt, K, r;
    float* pair;                 // out [M][K][K]
};

struct PairSmem {
    __attribute__((aligned(16))) float As[64][kPitch];
    __attribute__((aligned(16))) float Bs[64][kPitch];
    int64_t prev_row[64], cand_row[64];
    float red[kPairThreads / 64];
};

// S of position p of request req, whose rows start at row a (row m = a + p), into pair[m];
// by a workgroup of kPairThreads threads (eight waves: two per 32 x 32 quadrant of S, one
// per half of the rank).
__device__ __forceinline__ void pair_position(const PairArgs& A, int req, int a, int p, PairSmem& s) {
    const int tid = threadIdx.x;
    const int m = a + p;
    const int K = A.K, r = A.r, Vt = A.Vt, H = A.H;
    const int Jn = (p == 0) ? 1 : K;
    if (tid < 64) {
        const int64_t prev = (p == 0) ? A.last_tok[req] : (tid < K ? A.cand_tok[(int64_t)(m - 1) * K + tid] : 0);
        s.prev_row[tid] = clamp_tok(prev, Vt) * r;
        const int64_t cand = tid < K ? A.cand_tok[(int64_t)m * K + tid] : 0;
        s.cand_row[tid] = clamp_tok(cand, Vt) * r;
    }
    if (A.gate_w) {
        // w . h_p: eight consecutive elements per thread and round, the loads of every round
        // issued before the first product (one round trip for H up to 8192), then a fixed
        // tree over the lanes and the waves
        const uint16_t* h = A.hidden + (int64_t)m * H;
        float part = 0.f;
        if ((H & 7) == 0 && (reinterpret_cast<uintptr_t>(A.gate_w) & 15) == 0 &&
            (reinterpret_cast<uintptr_t>(h) & 15) == 0) {
            for (int base = 0; base < H; base += 8 * kPairThreads * kGateRounds) {
                u32x4 hv[kGateRounds];
                f32x4 ga[kGateRounds], gb[kGateRounds];
#pragma unroll
                for (int u = 0; u < kGateRounds; ++u) {
                    const int i = base + 8 * (tid + u * kPairThreads);
                    const bool ok = i < H;
                    hv[u] = ok ? *reinterpret_cast<const u32x4*>(h + i) : u32x4{0u, 0u, 0u, 0u};
                    ga[u] = ok ? *reinterpret_cast<const f32x4*>(A.gate_w + i) : f32x4{0.f, 0.f, 0.f, 0.f};
                    gb[u] = ok ? *reinterpret_cast<const f32x4*>(A.gate_w + i + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int u = 0; u < kGateRounds; ++u) {
                    const float wv[8] = {ga[u][0], ga[u][1], ga[u][2], ga[u][3], gb[u][0], gb[u][1], gb[u][2], gb[u][3]};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {   // a dword holds elements 2 e (low half) and 2 e + 1
                        part += wv[2 * e] * __uint_as_float(hv[u][e] << 16);
                        part += wv[2 * e + 1] * __uint_as_float(hv[u][e] & 0xFFFF0000u);
                    }
                }
            }
        } else {
            for (int i = tid; i < H; i += kPairThreads) part += A.gate_w[i] * bf16_bits_to_float(h[i]);
        }
        part = wave_sum(part);
        if ((tid & 63) == 0) s.red[tid >> 6] = part;
    }
    __syncthreads();
    float g = 1.f;
    if (A.gate_w) {
        static_assert(kPairThreads == 512, "eight wave sums");
        const float x = ((s.red[0] + s.red[1]) + (s.red[2] + s.red[3])) + ((s.red[4] + s.red[5]) + (s.red[6] + s.red[7]));
        g = 1.f / (1.f + expf(-x));
    }

    const float* TA = A.tables;
    const float* TB = A.tables + (int64_t)Vt * r;
    // waves w and w + 4 compute the 32 x 32 quadrant (jt, kt) = ((w % 4) / 2, w % 2) of S
    // on the matrix cores (v_mfma_f32_32x32x2_f32, fp32 products and sums), over the first
    // and the second half of every rank slice: in MFMA step s lane l supplies
    // A[prev 32 jt + l % 32][k] and B[cand 32 kt + l % 32][k] with k = 8 (s / 4) + 4 (l / 32)
    // + s % 4, the same in both, read as float4 from the LDS rows; the two partial sums
    // are added once at the end (first half + second half)
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lh = lane >> 5;
    const int quad = wv & 3, half = wv >> 2;
    const int jt = quad >> 1, kt = quad & 1;
    f32x16 acc = f32x16{};

    // With r % 4 == 0 and 16-byte aligned tables every row is read as float4, and a slice
    // arrives in four phases of 64 rank elements, two phases in flight at a time: the gather
    // of later phases runs while the MFMAs of earlier ones do.  Phase h holds groups 8 h ..
    // 8 h + 7; the first-half waves take groups below gmid and the second-half waves the
    // rest, each in ascending order, so every wave forms the same sums, in the same order,
    // as with the whole slice landed first.
    const bool vec = (r & 3) == 0 && (reinterpret_cast<uintptr_t>(A.tables) & 15) == 0;
    for (int i0 = 0; i0 < r; i0 += kRankSlice) {
        const int w = min(kRankSlice, r - i0);        // rank elements of this slice
        const int w8 = (w + 7) >> 3;                  // elements past w are zero in both operands
        const int gmid = (w8 + 1) >> 1;
        const float* arow = &s.As[32 * jt + lr][4 * lh];
        const float* brow = &s.Bs[32 * kt + lr][4 * lh];
        auto mfma_groups = [&](int g0, int g1) __attribute__((always_inline)) {
            for (int gi = g0; gi < g1; ++gi) {
                const f32x4 av = *reinterpret_cast<const f32x4*>(arow + 8 * gi);
                const f32x4 bv = *reinterpret_cast<const f32x4*>(brow + 8 * gi);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bv[e], acc, 0, 0, 0);
            }
        };
        if (vec) {
            constexpr int kPhases = 4;
            constexpr int kPer = 2 * 64 * (kRankSlice / kPhases) / 4 / kPairThreads;   // float4 per thread and phase
            static_assert(kRankSlice == 256 && kPer == 4, "phases of 64 rank elements");
            // float4 i of a thread in phase h: operand i / 2 (A, B), row tid / 16 + 32 (i % 2),
            // elements 64 h + 4 (tid % 16) .. + 3 (16 threads read the 256 contiguous bytes of a
            // row's phase).  Every load is issued (a row or element past the operand reads the
            // row's first element and is replaced by zero), so that the waits count loads.
            const float* rp[kPer];
            bool rok[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int b = i >> 1, row = (tid >> 4) + 32 * (i & 1);
                rok[i] = row < (b ? K : Jn);
                rp[i] = b ? TB + (rok[i] ? s.cand_row[row] : 0) : TA + (rok[i] ? s.prev_row[row] : 0);
            }
            f32x4 v[2][kPer];
            auto load = [&](int h, f32x4 (&dst)[kPer]) __attribute__((always_inline)) {
                const int c = 64 * h + 4 * (tid & 15);
#pragma unroll
                for (int i = 0; i < kPer; ++i)
                    dst[i] = *reinterpret_cast<const f32x4*>(rp[i] + i0 + (rok[i] && c < w ? c : 0));
            };
            load(0, v[0]);
            __builtin_amdgcn_sched_barrier(0);   // phase 0 issued first, so that its wait leaves phase 1 in flight
            load(1, v[1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < kPhases; ++h) {
                const int c = 64 * h + 4 * (tid & 15);
#pragma unroll
                for (int i = 0; i < kPer; ++i) {
                    const int b = i >> 1, row = (tid >> 4) + 32 * (i & 1);
                    const bool ok = rok[i] && c < w;
                    *reinterpret_cast<f32x4*>(b ? &s.Bs[row][c] : &s.As[row][c]) =
                        ok ? v[h & 1][i] : f32x4{0.f, 0.f, 0.f, 0.f};
                }
                __syncthreads();
                if (h + 2 < kPhases) load(h + 2, v[h & 1]);
                __builtin_amdgcn_sched_barrier(0);
                if (half) mfma_groups(max(8 * h, gmid), min(8 * h + 8, w8));
                else mfma_groups(8 * h, min(8 * h + 8, gmid));
            }
        } else {
            for (int f = tid; f < 2 * 64 * kRankSlice; f += kPairThreads) {
                const int b = f / (64 * kRankSlice), row = (f / kRankSlice) & 63, c = f % kRankSlice;
                const bool ok = row < (b ? K : Jn) && c < w;
                const float v = ok ? (b ? TB[s.cand_row[row] + i0 + c] : TA[s.prev_row[row] + i0 + c]) : 0.f;
                if (b) s.Bs[row][c] = v; else s.As[row][c] = v;
            }
            __syncthreads();
            if (half) mfma_groups(gmid, w8); else mfma_groups(0, gmid);
        }
        __syncthreads();
    }

    // the second-half waves hand their sums to the first-half waves through LDS (As is
    // free after the last slice's barrier): register i of lane l at float 1024 quad + 64 i + l
    float* xch = &s.As[0][0];
    if (half) {
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[1024 * quad + 64 * i + lane] = acc[i];
    }
    __syncthreads();
    if (half) return;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] += xch[1024 * quad + 64 * i + lane];

    // register i of lane l: S[32 jt + 8 (i / 4) + 4 (l / 32) + i % 4][32 kt + l % 32]
    float* out = A.pair + (int64_t)m * K * K;
    const int k = 32 * kt + lr;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int j = 32 * jt + 8 * (i / 4) + 4 * lh + i % 4;
        if (j < K && k < K) out[(int64_t)j * K + k] = (j < Jn) ? g * acc[i] : 0.f;
    }
}

struct WalkArgs {
    const int64_t* cand_tok;     // [M][K]
    const float* unary;          // [M][K]
    const float* pair;           // [M][K][K]
    const int32_t* row_offsets;  // [R+1] or null
    int L, M, K, walk;           // walk: DFLASH_WALK_VITERBI, DFLASH_WALK_GREEDY or kWalkSampled
    const double* uniforms;      // [M] (sampled)
    float temperature;           // (sampled)
    int64_t* tokens;             // out [M]
    float* scores;               // out [R]
    int32_t* slots;              // out [M] or null
    double* qprob;               // out [M][K] or null (sampled)
};

struct WalkSmem {
    __attribute__((aligned(16))) float Ss[2][kWalkChunk][64 * 64];
    float Us[2][kWalkChunk][64];
    float qbest[2][4][64];
    int qarg[2][4][64];
    uint8_t back[DFLASH_MAX_BLOCK_LEN][64];
    int path[DFLASH_MAX_BLOCK_LEN];
    float s_score;
};

// One Viterbi position p >= 1 by the four waves: wave q takes the best delta(j) + S[j][k]
// over its quarter j in [16 q, 16 q + 16) (svq[t] = S[16 q + t][k] in lane k, u = u_p[k]),
// then after one barrier the four quarters are combined in order (strict >), so the lowest
// j reaching the maximum wins; delta is updated in place and lane k's back-pointer returned.
// Every wave holds the same delta, lane k holding delta(k), and reads delta(j) by readlane.
__device__ __forceinline__ int viterbi_position(const float (&svq)[16], float us, int K, int q, int lane, float& d,
                                                int& par, WalkSmem& s) {
    const bool act = lane < K;
    float vv[16], dq[16];
    int jj[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) dq[t] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), 16 * q + t));
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int j = 16 * q + t;
        vv[t] = j < K ? dq[t] + svq[t] : -INFINITY;
        jj[t] = j;
    }
    // a tree over (value, j) in which the higher j wins only by strict >: the lowest j
    // reaching the maximum, as an ascending scan with strict > (slots past K are -inf)
#pragma unroll
    for (int w = 1; w < 16; w *= 2)
#pragma unroll
        for (int t = 0; t < 16; t += 2 * w)
            if (vv[t + w] > vv[t]) { vv[t] = vv[t + w]; jj[t] = jj[t + w]; }
    s.qbest[par][q][lane] = vv[0];
    s.qarg[par][q][lane] = jj[0];
    __syncthreads();
    float bb = s.qbest[par][0][lane];
    int ar = s.qarg[par][0][lane];
#pragma unroll
    for (int qq = 1; qq < 4; ++qq)
        if (s.qbest[par][qq][lane] > bb) { bb = s.qbest[par][qq][lane]; ar = s.qarg[par][qq][lane]; }
    if (bb == -INFINITY) ar = 0;   // nothing finite to extend: slot 0, as a scan from j = 0
    d = act ? us + bb : -INFINITY;
    par ^= 1;
    return min(ar, K - 1);
}

// The Viterbi walk of a block of at most NP positions with S, u, the candidates' target ids
// and the back-pointers in registers instead of LDS: lane k of wave q holds S_p[16 q + t][k]
// (t < 16), u_p[k] and the id of slot k of every position; the loads of position p + kAhead
// are issued as position p starts (at most 63 loads in flight per wave), so each position
// waits only for its own loads.  Clamped indices keep every load inside the request's rows;
// lanes and rows past K are masked.  The back-tracking reads the back-pointers by readlane
// (every wave holds the same ones); wave 0 writes tokens, slots and the score.
template <int NP>
__device__ __forceinline__ void viterbi_in_registers(const WalkArgs& A, int req, int a, int n, int q, int lane,
                                                     WalkSmem& s) {
    constexpr int kAhead = 3;   // 17 loads per position: three positions ahead stay under 63
    const int K = A.K, KK = K * K;
    const bool act = lane < K;
    const int kc = act ? lane : K - 1;
    // a wave-uniform base and 32-bit byte offsets: one address register per load
    auto at = [](const float* base, uint32_t i) __attribute__((always_inline)) {
        return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + (i << 2));
    };
    int64_t ct[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) ct[p] = A.cand_tok[(int64_t)(a + (p < n ? p : n - 1)) * K + kc];
    float sv[NP][16], uv[NP];
    auto load = [&](int p) __attribute__((always_inline)) {
        const int pc = p < n ? p : n - 1;
        const float* Sp = A.pair + (int64_t)(a + pc) * KK;
        uv[p] = at(A.unary + (int64_t)(a + pc) * K, (uint32_t)kc);
#pragma unroll
        for (int t = 0; t < 16; ++t) sv[p][t] = at(Sp, (uint32_t)(min(16 * q + t, K - 1) * K + kc));
        __builtin_amdgcn_sched_barrier(0);
    };
    const float s0 = A.pair[(int64_t)a * KK + kc];   // S_0[0][k]: the row of the token before the block
    uv[0] = A.unary[(int64_t)a * K + kc];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 1; p <= kAhead && p < NP; ++p) load(p);
    float d = act ? uv[0] + s0 : -INFINITY;
    int par = 0;
    int bk[NP];
#pragma unroll
    for (int p = 1; p < NP; ++p) {
        if (p + kAhead < NP) load(p + kAhead);
        bk[p] = p < n ? viterbi_position(sv[p], uv[p], K, q, lane, d, par, s) : 0;
    }
    const float score = wave_max(d);
    // NaN scores match no lane: fall back to slot 0 rather than index past the slots
    int c = min(lowest_lane(act && d == score), K - 1);
    int64_t tok = 0;
    int slot = 0;
#pragma unroll
    for (int p = NP - 1; p >= 0; --p) {
        if (p < n) {
            const int64_t t = ((int64_t)__builtin_amdgcn_readlane((int)(ct[p] >> 32), c) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)ct[p], c);
            if (lane == p) { tok = t; slot = c; }
            if (p > 0) c = __builtin_amdgcn_readlane(bk[p], c);
        }
    }
    if (q == 0) {
        if (lane == 0) A.scores[req] = score;
        if (lane < n) {
            A.tokens[a + lane] = tok;
            if (A.slots) A.slots[a + lane] = slot;
        }
    }
}

// The walk of request req through its lattice; writes tokens, scores (and slots, q).
__device__ __forceinline__ void walk_request(const WalkArgs& A, int req, WalkSmem& s) {
    const int tid = threadIdx.x;
    const int lane = tid & 63, q = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform quarter
    const int K = A.K, walk = A.walk;
    int a, n;
    row_range(A.row_offsets, req, A.L, A.M, a, n);
    if (n <= 0) {
        if (tid == 0) A.scores[req] = 0.f;
        return;
    }
    const bool act = lane < K;
    const int KK = K * K;
    const bool vec = K == 64 && (reinterpret_cast<uintptr_t>(A.pair) & 15) == 0;

    // Staging of positions c0 .. c0 + cn into buffer `buf`.  With K = 64 every thread
    // moves 16 float4 of S (one chunk = 4 x 16 KB): the loads of chunk c + 1 are issued
    // before chunk c is walked and stored after it.
    f32x4 sv[kWalkChunk * 4];
    float uv = 0.f;
    auto load_chunk = [&](int c0) {
        const int cn = min(kWalkChunk, n - c0);
        const f32x4* src = reinterpret_cast<const f32x4*>(A.pair + (int64_t)(a + c0) * KK);
        // u first: whatever wait its register needs then covers no load of S
        uv = tid < cn * K ? A.unary[(int64_t)(a + c0) * K + tid] : 0.f;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kWalkChunk * 4; ++i) {
            const int e = tid + i * kLatThreads;
            if (e < cn * 1024) sv[i] = src[e];
        }
    };
    auto store_chunk = [&](int c0, int buf) {
        const int cn = min(kWalkChunk, n - c0);
#pragma unroll
        for (int i = 0; i < kWalkChunk * 4; ++i) {
            const int e = tid + i * kLatThreads;
            if (e < cn * 1024) reinterpret_cast<f32x4*>(&s.Ss[buf][0][0])[e] = sv[i];
        }
        if (tid < cn * K) s.Us[buf][tid / K][tid % K] = uv;
        // every load of the chunk has landed, on every path through the stores above, so the
        // loads of the next chunk need not wait for these registers
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    };
    auto stage_generic = [&](int c0, int buf) {
        const int cn = min(kWalkChunk, n - c0);
        const float* src = A.pair + (int64_t)(a + c0) * KK;
        for (int e = tid; e < cn * KK; e += kLatThreads) {
            const int pp = e / KK, o = e - pp * KK;
            s.Ss[buf][pp][(o / K) * 64 + (o % K)] = src[e];
        }
        for (int e = tid; e < cn * K; e += kLatThreads) s.Us[buf][e / K][e % K] = A.unary[(int64_t)(a + c0) * K + e];
    };

    // Viterbi: every wave keeps delta of the previous position in lane k (d); a block of at
    // most kRegPositions positions keeps S and u in registers, a longer one (and the other
    // walks) stages kWalkChunk positions at a time in LDS
    float d = -INFINITY;
    int prev = 0;            // greedy: slot of the previous position (wave 0)
    float total = 0.f;       // greedy: running score (wave 0)
    int par = 0;             // parity of the qbest buffers
    if (walk == DFLASH_WALK_VITERBI && n <= kRegPositions) {
        if (n <= kRegPositions / 2) viterbi_in_registers<kRegPositions / 2>(A, req, a, n, q, lane, s);
        else viterbi_in_registers<kRegPositions>(A, req, a, n, q, lane, s);
        return;
    }
    if (vec) { load_chunk(0); store_chunk(0, 0); } else { stage_generic(0, 0); }
    __syncthreads();
    for (int c0 = 0, buf = 0; c0 < n; c0 += kWalkChunk, buf ^= 1) {
        const int cn = min(kWalkChunk, n - c0);
        const bool more = c0 + kWalkChunk < n;
        if (more && vec) load_chunk(c0 + kWalkChunk);
        for (int pp = 0; pp < cn; ++pp) {
            const int p = c0 + pp;
            if (walk == DFLASH_WALK_VITERBI) {
                if (p == 0) {
                    d = act ? s.Us[buf][0][lane] + s.Ss[buf][0][lane] : -INFINITY;
                } else {
                    // the 16 S entries of this quarter and u first (LDS reads that do not depend
                    // on delta)
                    float svq[16];
#pragma unroll
                    for (int t = 0; t < 16; ++t) svq[t] = s.Ss[buf][pp][(16 * q + t) * 64 + lane];
                    const int bp = viterbi_position(svq, s.Us[buf][pp][lane], K, q, lane, d, par, s);
                    if (q == 0) s.back[p][lane] = (uint8_t)bp;
                }
            } else if (walk == kWalkSampled) {
                if (tid < 64) {
                    // the row after the slot drawn before, in fp32; float weights (the fp32
                    // rounding of exp, taken in double); running and total sums in double in
                    // slot order; the smallest slot whose running sum exceeds U * total
                    const float v = act ? s.Us[buf][pp][lane] + s.Ss[buf][pp][prev * 64 + lane] : -INFINITY;
                    const float xs = act ? v / A.temperature : -INFINITY;
                    const float mx = wave_max(xs);
                    const float wf = act ? (float)exp((double)(xs - mx)) : 0.f;
                    // one sequential pass in slot order: lane k keeps the running sum W_k, and
                    // W_{K-1} is the total; the draw is the lowest lane with U * total < W_k
                    double run = 0.0, mine = 0.0;
                    for (int k = 0; k < K; ++k) {
                        run += (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(wf), k));
                        mine = lane == k ? run : mine;
                    }
                    const double tot = run;
                    const double thr = A.uniforms[a + p] * tot;
                    const int c = min(lowest_lane(act && thr < mine), K - 1);
                    if (A.qprob && act) A.qprob[(int64_t)(a + p) * K + lane] = (double)wf / tot;
                    total += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), c));
                    if (lane == 0) s.path[p] = c;
                    prev = c;
                }
            } else if (tid < 64) {
                const float v = act ? s.Us[buf][pp][lane] + s.Ss[buf][pp][prev * 64 + lane] : -INFINITY;
                const float mx = wave_max(v);
                const int c = min(lowest_lane(act && v == mx), K - 1);
                total += mx;
                if (lane == 0) s.path[p] = c;
                prev = c;
            }
        }
        if (more) {
            __syncthreads();    // everyone is done with buffer buf ^ 1 (walked two chunks ago)
            if (vec) store_chunk(c0 + kWalkChunk, buf ^ 1); else stage_generic(c0 + kWalkChunk, buf ^ 1);
            __syncthreads();
        }
    }
    if (tid < 64) {
        float score;
        if (walk == DFLASH_WALK_VITERBI) {
            score = wave_max(d);
            // NaN scores match no lane: fall back to slot 0 rather than index past the slots
            const int last = min(lowest_lane(act && d == score), K - 1);
            if (lane == 0) {
                int c = last;
                for (int p = n - 1; p >= 0; --p) {
                    s.path[p] = c;
                    if (p > 0) c = min((int)s.back[p][c], K - 1);
                }
            }
        } else {
            score = total;
        }
        if (lane == 0) s.s_score = score;
    }
    __syncthreads();
    if (tid == 0) A.scores[req] = s.s_score;
    for (int p = tid; p < n; p += kLatThreads) {
        const int c = s.path[p];
        A.tokens[a + p] = A.cand_tok[(int64_t)(a + p) * K + c];
        if (A.slots) A.slots[a + p] = c;
    }
}

}  // namespace

}  // namespace dflash
