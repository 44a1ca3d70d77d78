// Parts 3 and 4 of the draft step: the Markov-head candidate scorer over the
// packed Top-K lattice and the walk through it.
//
// Scorer (optimum-intel page "Export DFlash v2 and DSpark drafts ...", What
// does this PR do?: the Top-K lattice of the DSpark head, with transitions
// gated by the draft hidden states for DFlash v2; openvino.genai page "Add
// DSpark and DFlash v2 drafts ...", commit "DFlash-2 Markov head /
// BlockRowSource": one run over the packed block rows of all requests):
//   S_p[j][k] = g_p * <A[t_{p-1}[j]], B[t_p[k]]>,  S_0[0][k] = g_0 * <A[last], B[t_0[k]]>,
//   g_p = sigmoid(w . h_p) when gated, else 1.
// One workgroup per (position, request).  The K rows of A and of B it needs
// are gathered from the fp32 tables in 64-wide slices of the rank, stored
// transposed in LDS, and every thread accumulates a 4 x 4 block of S in a
// fixed order over the rank.
//
// Walk (same commit: the greedy walk takes the best candidate after the token
// before; the max-score walk is its Viterbi form): one wave per request, lane k
// owns slot k.  Viterbi keeps delta(k) in a register; delta(j) reaches every
// lane through readlane; back-pointers (lowest j at a tie) sit in LDS.  The
// argmax of a position is a DPP max reduction and the lowest lane of a ballot.

#include "common.hpp"
#include "internal.hpp"
#include "../../include/dflash_draft.h"

#include <math.h>

namespace dflash {

namespace {

constexpr int kPairThreads = 256;
constexpr int kSlice = 64;        // rank elements per LDS slice
constexpr int kPad = 68;          // padded LDS row (floats): aligned float4 reads

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

__global__ void __launch_bounds__(kPairThreads) pair_scores_kernel(
    const int64_t* __restrict__ cand_tok, const float* __restrict__ tables, const float* __restrict__ gate_w,
    const uint16_t* __restrict__ hidden, const int64_t* __restrict__ last_tok,
    const int32_t* __restrict__ row_offsets, int L, int M, int H, int Vt, int K, int r,
    float* __restrict__ pair) {
    __shared__ __attribute__((aligned(16))) float As[kSlice][kPad];
    __shared__ __attribute__((aligned(16))) float Bs[kSlice][kPad];
    __shared__ int64_t prev_row[64], cand_row[64];
    __shared__ float red[4];

    const int p = blockIdx.x, req = blockIdx.y;
    const int tid = threadIdx.x;
    int a, n;
    row_range(row_offsets, req, L, M, a, n);
    if (p >= n) return;
    const int m = a + p;

    float g = 1.f;
    if (gate_w) {
        float part = 0.f;
        const uint16_t* h = hidden + (int64_t)m * H;
        for (int i = tid; i < H; i += kPairThreads) part += gate_w[i] * bf16_bits_to_float(h[i]);
        part = wave_sum(part);
        if ((tid & 63) == 0) red[tid >> 6] = part;
        __syncthreads();
        const float x = (red[0] + red[1]) + (red[2] + red[3]);
        g = 1.f / (1.f + expf(-x));
    }

    const int Jn = (p == 0) ? 1 : K;
    if (tid < 64) {
        const int64_t prev = (p == 0) ? last_tok[req] : (tid < K ? cand_tok[(int64_t)(m - 1) * K + tid] : 0);
        prev_row[tid] = clamp_tok(prev, Vt) * r;
        const int64_t cand = tid < K ? cand_tok[(int64_t)m * K + tid] : 0;
        cand_row[tid] = clamp_tok(cand, Vt) * r;
    }
    __syncthreads();

    const float* TA = tables;
    const float* TB = tables + (int64_t)Vt * r;
    const int tj = tid >> 4, tk = tid & 15;
    float acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = 0.f;

    // Gather of one 64-wide rank slice: row `row` of A (previous tokens) and of B
    // (candidates), elements i0 .. i0+63.  With r % 4 == 0 the rows are 16-byte
    // aligned and every thread loads 4 float4 of A and 4 of B; the next slice is
    // in flight while the current one is multiplied.
    const bool vec = (r & 3) == 0 && (reinterpret_cast<uintptr_t>(tables) & 15) == 0;
    f32x4 ra[4], rb[4];
    auto gather = [&](int i0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int f4 = tid + i * kPairThreads;          // 0 .. 1023
            const int row = f4 >> 4, c = (f4 & 15) * 4;     // 16 float4 per 64-wide row slice
            f32x4 va = {0.f, 0.f, 0.f, 0.f}, vb = {0.f, 0.f, 0.f, 0.f};
            if (vec) {
                if (row < Jn && i0 + c < r) va = *reinterpret_cast<const f32x4*>(TA + prev_row[row] + i0 + c);
                if (row < K && i0 + c < r) vb = *reinterpret_cast<const f32x4*>(TB + cand_row[row] + i0 + c);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (row < Jn && i0 + c + e < r) va[e] = TA[prev_row[row] + i0 + c + e];
                    if (row < K && i0 + c + e < r) vb[e] = TB[cand_row[row] + i0 + c + e];
                }
            }
            ra[i] = va;
            rb[i] = vb;
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int f4 = tid + i * kPairThreads;
            const int row = f4 >> 4, c = (f4 & 15) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                As[c + e][row] = ra[i][e];
                Bs[c + e][row] = rb[i][e];
            }
        }
    };

    gather(0);
    for (int i0 = 0; i0 < r; i0 += kSlice) {
        stash();
        __syncthreads();
        if (i0 + kSlice < r) gather(i0 + kSlice);
#pragma unroll 8
        for (int ii = 0; ii < kSlice; ++ii) {
            const f32x4 av = *reinterpret_cast<const f32x4*>(&As[ii][4 * tj]);
            const f32x4 bv = *reinterpret_cast<const f32x4*>(&Bs[ii][4 * tk]);
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(av[x], bv[y], acc[x][y]);
        }
        __syncthreads();
    }

    float* out = pair + (int64_t)m * K * K;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int j = 4 * tj + x;
        if (j >= K) continue;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            const int k = 4 * tk + y;
            if (k < K) out[(int64_t)j * K + k] = (j < Jn) ? g * acc[x][y] : 0.f;
        }
    }
}

__global__ void __launch_bounds__(64) walk_kernel(const int64_t* __restrict__ cand_tok,
                                                  const float* __restrict__ unary, const float* __restrict__ pair,
                                                  const int32_t* __restrict__ row_offsets, int L, int M, int K,
                                                  int walk, int64_t* __restrict__ tokens,
                                                  float* __restrict__ scores, int32_t* __restrict__ slots) {
    __shared__ uint8_t back[DFLASH_MAX_BLOCK_LEN][64];
    __shared__ int path[DFLASH_MAX_BLOCK_LEN];
    const int req = blockIdx.x, lane = threadIdx.x;
    int a, n;
    row_range(row_offsets, req, L, M, a, n);
    if (n <= 0) {
        if (lane == 0) scores[req] = 0.f;
        return;
    }
    const bool act = lane < K;
    float score;
    if (walk == DFLASH_WALK_VITERBI) {
        float d = act ? unary[(int64_t)a * K + lane] + pair[(int64_t)a * K * K + lane] : -INFINITY;
        // lane k needs column k of S_p (64 strided floats) and u_p[k]; the column of
        // position p+1 is loaded while position p is folded in
        float colA[64], colB[64];
        float uA = 0.f, uB = 0.f;
        auto load_col = [&](int p, float (&col)[64], float& u) {
            const int64_t m = a + p;
            const float* S = pair + m * K * K;
#pragma unroll
            for (int j = 0; j < 64; ++j) col[j] = (j < K && act) ? S[j * K + lane] : 0.f;
            u = act ? unary[m * K + lane] : 0.f;
        };
        auto fold = [&](int p, const float (&col)[64], float u) {
            float best = -INFINITY;
            int arg = 0;
#pragma unroll
            for (int j = 0; j < 64; ++j) {
                if (j < K) {
                    const float dj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), j));
                    const float v = dj + col[j];
                    if (v > best) { best = v; arg = j; }
                }
            }
            d = act ? u + best : -INFINITY;
            back[p][lane] = (uint8_t)arg;
        };
        if (n > 1) load_col(1, colA, uA);
        for (int p = 1; p < n; p += 2) {
            if (p + 1 < n) load_col(p + 1, colB, uB);
            fold(p, colA, uA);
            if (p + 1 < n) {
                if (p + 2 < n) load_col(p + 2, colA, uA);
                fold(p + 1, colB, uB);
            }
        }
        score = wave_max(d);
        // NaN scores match no lane: fall back to slot 0 rather than index past the slots
        const int last = min(lowest_lane(act && d == score), K - 1);
        __syncthreads();
        if (lane == 0) {
            int c = last;
            for (int p = n - 1; p >= 0; --p) {
                path[p] = c;
                if (p > 0) c = min((int)back[p][c], K - 1);
            }
        }
    } else {
        int prev = 0;
        float total = 0.f;
        for (int p = 0; p < n; ++p) {
            const int64_t m = a + p;
            const float v = act ? unary[m * K + lane] + pair[(m * K + prev) * K + lane] : -INFINITY;
            const float mx = wave_max(v);
            const int c = min(lowest_lane(act && v == mx), K - 1);
            total += mx;
            if (lane == 0) path[p] = c;
            prev = c;
        }
        score = total;
    }
    __syncthreads();
    if (lane == 0) scores[req] = score;
    for (int p = lane; p < n; p += 64) {
        const int c = path[p];
        tokens[a + p] = cand_tok[(int64_t)(a + p) * K + c];
        if (slots) slots[a + p] = c;
    }
}

}  // namespace

hipError_t launch_pair_scores(const int64_t* cand_tok, const float* tables, const float* gate_w,
                              const uint16_t* hidden, const int64_t* last_tok, const int32_t* row_offsets,
                              int R, int L, int M, int H, int Vt, int K, int r, float* pair, hipStream_t s) {
    if (R <= 0 || M <= 0) return hipSuccess;
    hipLaunchKernelGGL(pair_scores_kernel, dim3(L, R), dim3(kPairThreads), 0, s, cand_tok, tables, gate_w, hidden,
                       last_tok, row_offsets, L, M, H, Vt, K, r, pair);
    return hipGetLastError();
}

hipError_t launch_walk(const int64_t* cand_tok, const float* unary, const float* pair, const int32_t* row_offsets,
                       int R, int L, int M, int K, int walk, int64_t* tokens, float* scores, int32_t* slots,
                       hipStream_t s) {
    if (R <= 0) return hipSuccess;
    hipLaunchKernelGGL(walk_kernel, dim3(R), dim3(64), 0, s, cand_tok, unary, pair, row_offsets, L, M, K, walk,
                       tokens, scores, slots);
    return hipGetLastError();
}

}  // namespace dflash
