// Part 2 of the draft step as stand-alone kernels: the Top-K of every row
// (the row's device function is in topk_row.hpp), the streaming pass that
// computes tile maxima of logits from elsewhere, and the head-less argmax.

#include "common.hpp"
#include "internal.hpp"
#include "topk_row.hpp"

#include <math.h>

namespace dflash {

namespace {

__global__ void __launch_bounds__(kThreads) topk_tiles_kernel(TopkRowArgs a) {
    __shared__ TopkSmem s;
    topk_row(a, blockIdx.x, s);
}

// The bound of the lm_head's logits filter: tau[m] = the K-th largest of the n sample logits
// of row m (the exact logits of sampled vocabulary tiles), the last slot of their top K.
__global__ void __launch_bounds__(kThreads) sample_tau_kernel(const float* __restrict__ zs, int64_t ldzs, int n,
                                                              int K, float* __restrict__ tau) {
    __shared__ ChunkShared sh;
    __shared__ uint64_t top[kMaxTopK];
    const int m = blockIdx.x;
    chunk_select<16>(zs + (int64_t)m * ldzs, 0, n, K, top, sh);
    if (threadIdx.x == 0) tau[m] = key_to_float(entry_key(top[K - 1]));
}

}  // namespace

// ---------------------------------------------------------------- head-less argmax
// f(z) = cap tanh(scale z / cap) (cap > 0) or scale z, as head_apply computes it, is
// non-decreasing, so every logit with f(z) = max f lies in a tile whose maximum m_t has
// f(m_t) = max f: with tile maxima only those tiles are read.  Ties go to the lowest id.

// (value, id) with the larger value, the lower id on a tie.
__device__ __forceinline__ void better(float& v, int& i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__global__ void __launch_bounds__(kThreads) argmax_kernel(const float* __restrict__ logits, int64_t ldz,
                                                          const float* __restrict__ tmax, int64_t ldt, int V,
                                                          float scale, float cap, const int64_t* __restrict__ d2t,
                                                          int64_t* __restrict__ tokens, float* __restrict__ values) {
    __shared__ float tf[kTileCap];     // z' of the tile maxima (rows of at most kTileCap tiles)
    __shared__ int sel[kSelCap];
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    __shared__ int s_best, s_nsel;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int m = blockIdx.x;
    const float* row = logits + (int64_t)m * ldz;
    const HeadMap hm = head_map(scale, cap);
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    // block-wide (max, lowest id)
    auto reduce = [&]() {
        for (int o = 32; o > 0; o >>= 1) {
            const float v2 = __shfl_xor(bv, o);
            const int i2 = __shfl_xor(bi, o);
            better(bv, bi, v2, i2);
        }
        __syncthreads();
        if (lane == 0) { s_v[w] = bv; s_i[w] = bi; }
        __syncthreads();
        bv = s_v[0]; bi = s_i[0];
        for (int q = 1; q < 4; ++q) better(bv, bi, s_v[q], s_i[q]);
    };
    // every logit of the row, sixteen loads in flight per thread at a time
    auto scan_row = [&]() {
        bv = -INFINITY;
        bi = 0x7fffffff;
        for (int base = 0; base < V; base += kThreads * 16) {
            float zv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int v = base + tid + kThreads * i;
                zv[i] = v < V ? row[v] : -INFINITY;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int v = base + tid + kThreads * i;
                if (v < V) better(bv, bi, head_apply(hm, zv[i]), v);
            }
        }
        reduce();
    };
    const int tiles = (V + 31) / 32;
    if (tmax && tiles <= kTileCap) {
        const float* trow = tmax + (int64_t)m * ldt;
        constexpr int kTPT = kTileCap / kThreads;
        float tv[kTPT];
#pragma unroll
        for (int i = 0; i < kTPT; ++i) {
            const int t = tid + kThreads * i;
            tv[i] = t < tiles ? trow[t] : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < kTPT; ++i) {
            const int t = tid + kThreads * i;
            if (t < tiles) {
                const float f = head_apply(hm, tv[i]);
                tf[t] = f;
                better(bv, bi, f, t);
            }
        }
        if (tid == 0) { s_best = 0x7fffffff; s_nsel = 0; }
        reduce();
        const float fmax = bv;
        // the tiles that reach fmax
        for (int t = tid; t < tiles; t += kThreads) {
            if (tf[t] == fmax) {
                const int i = atomicAdd(&s_nsel, 1);
                if (i < kSelCap) sel[i] = t;
            }
        }
        __syncthreads();
        const int nsel = s_nsel;
        if (nsel <= kSelCap) {
            for (int base = 0; base < nsel * 32; base += kThreads * 8) {
                float zv[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int e = base + tid + kThreads * i;
                    const int v = e < nsel * 32 ? sel[e >> 5] * 32 + (e & 31) : V;
                    zv[i] = v < V ? row[v] : -INFINITY;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int e = base + tid + kThreads * i;
                    const int v = e < nsel * 32 ? sel[e >> 5] * 32 + (e & 31) : V;
                    if (v < V && head_apply(hm, zv[i]) == fmax) atomicMin(&s_best, v);
                }
            }
            __syncthreads();
            bi = s_best;
            bv = fmax;
        } else {
            scan_row();   // heavy ties: every logit
        }
    } else {
        scan_row();
    }
    if (bi == 0x7fffffff) bi = 0;   // NaN rows match nothing: id 0
    if (tid == 0) {
        tokens[m] = d2t ? (int64_t)bi + d2t[bi] : (int64_t)bi;
        if (values) values[m] = bv;
    }
}

hipError_t launch_argmax(const float* logits, int64_t ldz, const float* tile_max, int64_t ldt, const int64_t* d2t,
                         int M, int V, float scale, float cap, int64_t* tokens, float* values, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(argmax_kernel, dim3(M), dim3(kThreads), 0, s, logits, ldz, ldt > 0 ? tile_max : nullptr, ldt,
                       V, scale, cap, d2t, tokens, values);
    return hipGetLastError();
}

int topk_tiles_chunks(int V) { return topk_chunks(V); }

hipError_t launch_sample_tau(const float* zs, int64_t ldzs, int n, int M, int K, float* tau, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (n > kThreads * 16 || n < K || (n & 3)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(sample_tau_kernel, dim3(M), dim3(kThreads), 0, s, zs, ldzs, n, K, tau);
    return hipGetLastError();
}

hipError_t launch_topk_tiles(const float* logits, int64_t ldz, const float* tile_max, int64_t ldt,
                             const float* lse, const float2* lse_part, int nparts, const int64_t* d2t, int M, int V,
                             int K, int32_t* cand_idx, int64_t* cand_tok, float* unary, hipStream_t s,
                             const uint8_t* tile_mask, const float* tau) {
    if (M <= 0) return hipSuccess;
    const TopkRowArgs a = topk_row_args(logits, ldz, tile_max, ldt, lse, lse_part, nparts, d2t, V, K, cand_idx,
                                        cand_tok, unary, tile_mask, tau);
    hipLaunchKernelGGL(topk_tiles_kernel, dim3(M), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

namespace {

// The maximum of every 32-logit tile of every row, in one streaming pass: eight
// lanes read a tile's 128 bytes with one 16-byte load each (a wave reads 1 KB of
// contiguous logits per instruction), eight tiles' loads in flight per thread,
// and the eight lanes combine their maxima with xor shuffles.
constexpr int kTmU = 8;               // loads in flight per thread
constexpr int kTmTiles = 32 * kTmU;   // tiles per workgroup
__global__ void __launch_bounds__(kThreads) tile_max_kernel(const float* __restrict__ logits, int64_t ldz, int V,
                                                            int tiles, float* __restrict__ tmax, int64_t ldt) {
    const int m = blockIdx.y;
    const float* row = logits + (int64_t)m * ldz;
    const int q8 = threadIdx.x & 7;
    const int t0 = blockIdx.x * kTmTiles + (threadIdx.x >> 3);
    f32x4 z[kTmU];
#pragma unroll
    for (int u = 0; u < kTmU; ++u) {
        const int t = t0 + 32 * u;
        const int v = t * 32 + 4 * q8;
        // a run of four starting inside the row ends inside its stride (ldz >= V, a multiple of 4)
        z[u] = (t < tiles && v < V) ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + v))
                                    : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
#pragma unroll
    for (int u = 0; u < kTmU; ++u) {
        const int t = t0 + 32 * u;
        const int v = t * 32 + 4 * q8;
        float mx = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; ++q) mx = fmaxf(mx, v + q < V ? z[u][q] : -INFINITY);
        mx = fmaxf(mx, __shfl_xor(mx, 1));
        mx = fmaxf(mx, __shfl_xor(mx, 2));
        mx = fmaxf(mx, __shfl_xor(mx, 4));
        if (q8 == 0 && t < tiles) tmax[(int64_t)m * ldt + t] = mx;
    }
}

}  // namespace

hipError_t launch_tile_max(const float* logits, int64_t ldz, int M, int V, float* tile_max, int64_t ldt,
                           hipStream_t s) {
    if (M <= 0) return hipSuccess;
    const int tiles = (V + 31) / 32;
    hipLaunchKernelGGL(tile_max_kernel, dim3((tiles + kTmTiles - 1) / kTmTiles, M), dim3(kThreads), 0, s, logits,
                       ldz, V, tiles, tile_max, ldt);
    return hipGetLastError();
}

}  // namespace dflash
