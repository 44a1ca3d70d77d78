// The dense Markov walk (openvino.genai page "Add DSpark and DFlash v2 drafts
// ...", Description: with markov_head_top_k = 0, DSpark only, the head
// corrects every drafted position, one inference per position; commit
// "DFlash-2 Markov head / BlockRowSource": a dense Markov step biases the
// scaled rows by the token drafted before, and a greedy request takes the
// best biased token).  For request r at position p, with s_0 the last
// accepted token and s_{p+1} = t(c_p):
//   x_p[v] = f(z_m[v]) + <A[s_p], B[t(v)]>,   c_p = the lowest v maximizing x_p,
// f the scale and soft cap of the head-less rows, t(v) = v + d2t[v].
//
// One launch per position (the next position needs every request's choice).
// A workgroup takes 256 vocabulary ids for up to kGroup requests; the biases
// are a small fp32 GEMM (requests x ids x rank) on the matrix cores; (x, id)
// per request reduces to one packed 64-bit entry (order-preserving key of x << 32 | ~id, so the maximum
// entry is the largest x with the lowest id); one atomicMax per request and
// workgroup merges the workgroups.

#include "common.hpp"
#include "internal.hpp"

#include <math.h>

namespace dflash {

namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 32;     // requests per workgroup
constexpr int kRankChunk = 256; // rank elements of the A rows staged in LDS at a time
constexpr int kAStride = kRankChunk + 4;   // padded row stride: the 32 rows of a read hit distinct banks

__device__ __forceinline__ float head_scale_cap(float x, float scale, float cap) {
    return cap > 0.f ? cap * tanhf(scale * x / cap) : scale * x;
}

__device__ __forceinline__ void rows_of(const int32_t* row_offsets, int req, int L, int M, int& a, int& n) {
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

__device__ __forceinline__ int64_t target_of(int64_t v, const int64_t* d2t) { return d2t ? v + d2t[v] : v; }

__global__ void __launch_bounds__(kThreads) dense_clear_kernel(uint64_t* best, int n) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < n) best[i] = 0;
}

// One position for kGroup (32) requests and 256 vocabulary ids: wave w computes the
// 32 x 32 bias tiles of vocab tiles 2w and 2w + 1 with v_mfma_f32_32x32x2_f32
// (fp32 products and sums).  Operands: in MFMA step s lane l supplies A[l % 32][k]
// and B[k][l % 32] with k = 8 (s / 4) + 4 (l / 32) + s % 4, the same index in both,
// so every lane reads 4 consecutive rank elements per 4 steps.  Result register i
// of lane l is request 8 (i / 4) + 4 (l / 32) + i % 4 at vocab id l % 32 of the tile.
__global__ void __launch_bounds__(kThreads) dense_pos_kernel(
    const float* __restrict__ logits, int64_t ldz, const int64_t* __restrict__ d2t,
    const float* __restrict__ tables, const int64_t* __restrict__ last_tok, const int32_t* __restrict__ row_offsets,
    int R, int L, int M, int V, int Vt, int r, float scale, float cap, int p, uint64_t* __restrict__ best) {
    __shared__ __attribute__((aligned(16))) float As[kGroup * kAStride];   // a rank chunk of the A rows
    __shared__ int64_t arow[kGroup];
    __shared__ int mrow[kGroup];          // the request's row at position p, -1 when it has none
    __shared__ uint64_t wbest[4][kGroup];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int g0 = blockIdx.y * kGroup;
    const int ng = min(kGroup, R - g0);
    const float* TA = tables;
    const float* TB = tables + (int64_t)Vt * r;

    if (tid < kGroup) {
        int m = -1;
        int64_t s = 0;
        if (tid < ng) {
            const int req = g0 + tid;
            int a, n;
            rows_of(row_offsets, req, L, M, a, n);
            if (p < n) {
                m = a + p;
                if (p == 0) {
                    s = last_tok[req];
                } else {
                    const uint64_t e = best[(int64_t)(p - 1) * R + req];
                    s = target_of(min((int64_t)entry_id(e), (int64_t)V - 1), d2t);
                }
            }
        }
        s = s < 0 ? 0 : (s >= Vt ? (int64_t)Vt - 1 : s);
        arow[tid] = s * r;
        mrow[tid] = m;
    }
    __syncthreads();
    // the B rows of this lane's vocab ids in the wave's two tiles
    const int vt0 = blockIdx.x * kThreads + w * 64;   // first id of the wave's tiles
    const float* brow[2];
    bool bok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int v = vt0 + 32 * j + lr;
        bok[j] = v < V;
        int64_t t = bok[j] ? target_of(v, d2t) : 0;
        t = t < 0 ? 0 : (t >= Vt ? (int64_t)Vt - 1 : t);
        brow[j] = TB + t * r;
    }

    f32x16 acc[2] = {f32x16{}, f32x16{}};
    const bool vec = (r & 3) == 0 && (reinterpret_cast<uintptr_t>(tables) & 15) == 0;
    auto load_b = [&](int k0, int j) __attribute__((always_inline)) -> f32x4 {
        const int k = k0 + 4 * lh;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (vec) {
            if (bok[j] && k < r) x = *reinterpret_cast<const f32x4*>(brow[j] + k);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (bok[j] && k + e < r) ? brow[j][k + e] : 0.f;
        }
        return x;
    };
    auto step = [&](int kc, const f32x4 (&bv)[2]) __attribute__((always_inline)) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(&As[lr * kAStride + kc + 4 * lh]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bv[0][e], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bv[1][e], acc[1], 0, 0, 0);
        }
    };
    for (int c0 = 0; c0 < r; c0 += kRankChunk) {
        const int cn = min(kRankChunk, r - c0);
        const int cpad = (cn + 15) / 16 * 16;
        __syncthreads();   // the previous chunk's reads are done
        for (int e = tid; e < kGroup * cpad; e += kThreads) {
            const int q = e / cpad, i = e % cpad;
            As[q * kAStride + i] = (mrow[q] >= 0 && i < cn) ? TA[arow[q] + c0 + i] : 0.f;
        }
        __syncthreads();
        // B runs two 8-element groups ahead of the MFMAs
        f32x4 b0[2] = {load_b(c0, 0), load_b(c0, 1)};
        f32x4 b1[2] = {load_b(c0 + 8, 0), load_b(c0 + 8, 1)};
        for (int kc = 0; kc < cpad; kc += 16) {
            const f32x4 b2[2] = {load_b(c0 + kc + 16, 0), load_b(c0 + kc + 16, 1)};
            step(kc, b0);
            const f32x4 b3[2] = {load_b(c0 + kc + 24, 0), load_b(c0 + kc + 24, 1)};
            step(kc + 8, b1);
            b0[0] = b2[0]; b0[1] = b2[1];
            b1[0] = b3[0]; b1[1] = b3[1];
        }
    }

    // x = f(z) + bias per (request, id); per request the best (x, lowest id) of the block
    uint64_t e16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int q = 8 * (i / 4) + 4 * lh + i % 4;
        const int m = q < ng ? mrow[q] : -1;
        uint64_t best_e = 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int v = vt0 + 32 * j + lr;
            if (m >= 0 && v < V) {
                const float x = head_scale_cap(logits[(int64_t)m * ldz + v], scale, cap) + acc[j][i];
                const uint64_t en = pack_entry(float_to_key(x), (uint32_t)v);
                best_e = en > best_e ? en : best_e;
            }
        }
        // max over the 32 lanes that share lh (the 32 ids of the tile)
        for (int o = 16; o > 0; o >>= 1) {
            const uint64_t o2 = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(best_e >> 32), o) << 32) |
                                (uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)best_e, o);
            best_e = o2 > best_e ? o2 : best_e;
        }
        e16[i] = best_e;
    }
    if (lr == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) wbest[w][8 * (i / 4) + 4 * lh + i % 4] = e16[i];
    }
    __syncthreads();
    if (tid < ng && mrow[tid] >= 0) {
        uint64_t bb = wbest[0][tid];
        for (int k = 1; k < 4; ++k) bb = wbest[k][tid] > bb ? wbest[k][tid] : bb;
        atomicMax(reinterpret_cast<unsigned long long*>(&best[(int64_t)p * R + g0 + tid]), (unsigned long long)bb);
    }
}

__global__ void __launch_bounds__(kThreads) dense_finish_kernel(const uint64_t* __restrict__ best,
                                                                const int64_t* __restrict__ d2t,
                                                                const int32_t* __restrict__ row_offsets, int R,
                                                                int L, int M, int V, int64_t* __restrict__ tokens,
                                                                float* __restrict__ values) {
    const int i = blockIdx.x * kThreads + threadIdx.x;   // (position, request)
    if (i >= L * R) return;
    const int p = i / R, req = i % R;
    int a, n;
    rows_of(row_offsets, req, L, M, a, n);
    if (p >= n) return;
    const uint64_t e = best[i];
    const int64_t id = min((int64_t)entry_id(e), (int64_t)V - 1);
    tokens[a + p] = target_of(id, d2t);
    if (values) values[a + p] = key_to_float(entry_key(e));
}

}  // namespace

hipError_t launch_dense_walk(const float* logits, int64_t ldz, const int64_t* d2t, const float* tables,
                             const int64_t* last_tok, const int32_t* row_offsets, int R, int L, int M, int V,
                             int Vt, int r, float scale, float cap, uint64_t* best, int64_t* tokens, float* values,
                             hipStream_t s) {
    if (R <= 0 || M <= 0) return hipSuccess;
    const int nb = L * R;
    hipLaunchKernelGGL(dense_clear_kernel, dim3((nb + kThreads - 1) / kThreads), dim3(kThreads), 0, s, best, nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((V + kThreads - 1) / kThreads, (R + kGroup - 1) / kGroup);
    for (int p = 0; p < L; ++p) {
        hipLaunchKernelGGL(dense_pos_kernel, grid, dim3(kThreads), 0, s, logits, ldz, d2t, tables, last_tok,
                           row_offsets, R, L, M, V, Vt, r, scale, cap, p, best);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(dense_finish_kernel, dim3((nb + kThreads - 1) / kThreads), dim3(kThreads), 0, s, best, d2t,
                       row_offsets, R, L, M, V, tokens, values);
    return hipGetLastError();
}

}  // namespace dflash
