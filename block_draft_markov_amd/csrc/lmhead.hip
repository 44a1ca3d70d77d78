// Part 1 of the draft step: the lm_head projection z = W h over the draft
// vocabulary (optimum-intel page "Support MiniCPM-OCR-1.0-DSpark", What does
// this PR do?: the draft applies its own lm_head and outputs logits over the
// draft vocabulary), as a bf16 MFMA GEMM with fp32 accumulation, and a fused
// epilogue that keeps a running (max, sum exp(z - max)) per row so that the
// row's log-sum-exp needs no second pass over the logits.
//
// Shapes: hidden [M][H] bf16, W [V][H] bf16 (both contiguous along H),
// logits [M][ldz] fp32.  At the Qwen3-4B batch shape (M = 224, H = 2560,
// V = 151936) the kernel moves 778 MB of W for 174 GFLOP: 224 flop per byte
// of W, under the MI355X ridge of about 312, so it is bound by HBM; W is read
// exactly once.
//
// Work split.  The vocabulary is cut into tiles of 16 rows.  Workgroup b owns
// the contiguous tile range [b*T/G, (b+1)*T/G) and all 16*MT hidden rows of
// its row chunk; it walks its range in passes of 4*NT tiles (NT per wave).
// Every wave streams the W rows of its own tiles from HBM straight into MFMA
// operand registers (no reuse across waves, so no LDS), while the hidden tile
// that all four waves share is staged through LDS, double buffered.
//
// MFMA: v_mfma_f32_16x16x32_bf16 with A = W (16 vocab rows x 32 h), B = hidden
// (32 h x 16 rows).  The reduction index only has to be paired identically in
// A and B, so every lane loads 16 contiguous h values (two operands) per row
// and 64-element step: lane group g (lanes 16g..16g+15) of the MFMA of
// sub-step s covers h = k0 + 16 g + 8 s .. + 7 in both operands.  The result
// D[i][j] of a lane is 4 consecutive vocabulary entries (i = 4 (lane / 16) + q)
// of one row (j = lane % 16), stored as one 16-byte write.

#include "common.hpp"
#include "internal.hpp"

#include <math.h>

namespace dflash {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;                       // h elements per stage
constexpr int kRowBytes = kBK * 2 + 16;       // padded LDS row: conflict-free 16-byte reads
constexpr int kNT = 4;                        // vocab tiles per wave per pass

struct LmHeadArgs {
    const uint16_t* hidden;
    const uint16_t* W;
    float* logits;
    float2* part;
    int64_t ldz;
    int M, H, V;
    int tiles;   // ceil(V / 16)
    int G;       // workgroups along the vocabulary
};

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
    if (s2 == 0.f) return;
    if (s == 0.f) { m = m2; s = s2; return; }
    float mn = fmaxf(m, m2);
    s = s * expf(m - mn) + s2 * expf(m2 - mn);
    m = mn;
}

template <int MT, int NT>
__global__ void __launch_bounds__(kThreads) lmhead_gemm_lse_kernel(LmHeadArgs a) {
    constexpr int ROWS = MT * 16;
    constexpr int CHUNKS = ROWS * (kBK / 8);                  // 16-byte pieces of a hidden stage
    constexpr int PER_THREAD = (CHUNKS + kThreads - 1) / kThreads;
    __shared__ __attribute__((aligned(16))) uint8_t hs[2][ROWS][kRowBytes];
    __shared__ float2 wpart[4][ROWS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.x;
    const int m0 = blockIdx.y * ROWS;
    const int t_begin = (int)((int64_t)b * a.tiles / a.G);
    const int t_end = (int)((int64_t)(b + 1) * a.tiles / a.G);
    const int H = a.H;
    const int nks = (H + kBK - 1) / kBK;
    const int lr = lane & 15, lg = lane >> 4;

    float run_m = 0.f, run_s = 0.f;   // running LSE partial of row m0 + tid (s == 0: empty)

    // hidden stage ks -> registers
    auto load_h = [&](int ks, bf16x8 (&reg)[PER_THREAD]) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int c = tid + i * kThreads;
            const int row = c >> 3, col = ks * kBK + (c & 7) * 8;
            bf16x8 v = {};
            if (c < CHUNKS && m0 + row < a.M && col < H)
                v = *reinterpret_cast<const bf16x8*>(a.hidden + (int64_t)(m0 + row) * H + col);
            reg[i] = v;
        }
    };
    auto store_h = [&](int buf, const bf16x8 (&reg)[PER_THREAD]) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int c = tid + i * kThreads;
            if (c < CHUNKS)
                *reinterpret_cast<bf16x8*>(&hs[buf][c >> 3][(c & 7) * 16]) = reg[i];
        }
    };

    for (int pt = t_begin; pt < t_end; pt += 4 * NT) {
        const int npass = min(4 * NT, t_end - pt);
        const bf16x8* wrow[NT];
        bool tvalid[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int tloc = wave + 4 * j;
            tvalid[j] = tloc < npass;
            int v = (pt + tloc) * 16 + lr;
            v = min(v, a.V - 1);   // rows past the vocabulary load a valid row; their results are dropped
            wrow[j] = reinterpret_cast<const bf16x8*>(a.W + (int64_t)v * H);
        }
        auto load_w = [&](int ks, bf16x8 (&w)[NT][2]) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int col = ks * kBK + lg * 16 + s * 8;
                    bf16x8 v = {};
                    if (tvalid[j] && col < H) v = __builtin_nontemporal_load(wrow[j] + (col >> 3));
                    w[j][s] = v;
                }
            }
        };

        f32x4 acc[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        bf16x8 hreg[PER_THREAD];
        bf16x8 wcur[NT][2], wnext[NT][2];
        load_h(0, hreg);
        load_w(0, wcur);
        store_h(0, hreg);
        __syncthreads();

        for (int ks = 0; ks < nks; ++ks) {
            const int buf = ks & 1;
            const bool more = ks + 1 < nks;
            if (more) {
                load_h(ks + 1, hreg);
                load_w(ks + 1, wnext);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint8_t* rowp = &hs[buf][mt * 16 + lr][lg * 32];
                const bf16x8 h0 = *reinterpret_cast<const bf16x8*>(rowp);
                const bf16x8 h1 = *reinterpret_cast<const bf16x8*>(rowp + 16);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wcur[j][0], h0, acc[mt][j], 0, 0, 0);
                    acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wcur[j][1], h1, acc[mt][j], 0, 0, 0);
                }
            }
            if (more) store_h(buf ^ 1, hreg);
            __syncthreads();
            if (more) {
#pragma unroll
                for (int j = 0; j < NT; ++j) { wcur[j][0] = wnext[j][0]; wcur[j][1] = wnext[j][1]; }
            }
        }

        // ---- epilogue of the pass: store logits, fold the rows' (max, sum exp) partials
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = m0 + mt * 16 + lr;
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int v0 = (pt + wave + 4 * j) * 16 + lg * 4;
                const f32x4 z = acc[mt][j];
                if (tvalid[j] && m < a.M) {
                    float* dst = a.logits + (int64_t)m * a.ldz + v0;
                    if (v0 + 3 < a.V) {
                        *reinterpret_cast<f32x4*>(dst) = z;
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (v0 + q < a.V) dst[q] = z[q];
                    }
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (tvalid[j] && v0 + q < a.V) mx = fmaxf(mx, z[q]);
            }
            float sm = 0.f;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int v0 = (pt + wave + 4 * j) * 16 + lg * 4;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (tvalid[j] && v0 + q < a.V) sm += expf(acc[mt][j][q] - mx);
            }
            // the four lanes lr, lr+16, lr+32, lr+48 hold the same row
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const float m2 = __shfl_xor(mx, o);
                const float s2 = __shfl_xor(sm, o);
                lse_merge(mx, sm, m2, s2);
            }
            if (lg == 0) wpart[wave][mt * 16 + lr] = make_float2(mx, sm);
        }
        __syncthreads();
        if (tid < ROWS) {
#pragma unroll
            for (int w = 0; w < 4; ++w) lse_merge(run_m, run_s, wpart[w][tid].x, wpart[w][tid].y);
        }
        __syncthreads();
    }
    if (tid < ROWS && m0 + tid < a.M)
        a.part[(int64_t)(m0 + tid) * a.G + b] = make_float2(run_m, run_s);
}

template <int MT>
hipError_t launch_mt(const LmHeadArgs& a, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((lmhead_gemm_lse_kernel<MT, kNT>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

int row_tiles_per_chunk(int M) {
    if (M <= 0) return 1;
    const int gy = (M + 255) / 256;
    const int rows = (M + gy - 1) / gy;
    return (rows + 15) / 16;
}

// One (max, sum) partial per row and vocabulary workgroup -> lse.
__global__ void __launch_bounds__(64) lse_combine_kernel(const float2* part, int nparts, float* lse, int M) {
    const int m = blockIdx.x;
    const int lane = threadIdx.x;
    float mx = 0.f, sm = 0.f;
    for (int i = lane; i < nparts; i += 64) {
        const float2 p = part[(int64_t)m * nparts + i];
        lse_merge(mx, sm, p.x, p.y);
    }
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(mx, o);
        const float s2 = __shfl_xor(sm, o);
        lse_merge(mx, sm, m2, s2);
    }
    if (lane == 0) lse[m] = mx + logf(sm);
}

// lse of rows of given logits: a running (max, sum) per thread, merged in a fixed tree.
__global__ void __launch_bounds__(256) row_lse_kernel(const float* logits, int64_t ldz, float* lse, int V) {
    __shared__ float2 red[4];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const float* row = logits + (int64_t)m * ldz;
    float mx = -INFINITY;
    for (int v = tid; v < V; v += 256) mx = fmaxf(mx, row[v]);
    float sm = 0.f;
    for (int v = tid; v < V; v += 256) sm += expf(row[v] - mx);
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(mx, o);
        const float s2 = __shfl_xor(sm, o);
        lse_merge(mx, sm, m2, s2);
    }
    if ((tid & 63) == 0) red[tid >> 6] = make_float2(mx, sm);
    __syncthreads();
    if (tid == 0) {
        float a = 0.f, s = 0.f;
        for (int w = 0; w < 4; ++w) lse_merge(a, s, red[w].x, red[w].y);
        lse[m] = a + logf(s);
    }
}

}  // namespace

int lmhead_grid_y(int M) { return (M + 255) / 256; }

int lmhead_grid_x(int M, int V) {
    const int mt = row_tiles_per_chunk(M);
    const int tiles = (V + 15) / 16;
    const int per_pass = 4 * kNT;
    const int cap = mt <= 4 ? 1024 : (mt <= 8 ? 512 : 256);
    const int need = (tiles + per_pass - 1) / per_pass;
    return need < cap ? need : cap;
}

hipError_t launch_lmhead(const uint16_t* hidden, const uint16_t* W, float* logits, int64_t ldz,
                         float2* lse_part, int M, int H, int V, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    LmHeadArgs a;
    a.hidden = hidden; a.W = W; a.logits = logits; a.part = lse_part; a.ldz = ldz;
    a.M = M; a.H = H; a.V = V;
    a.tiles = (V + 15) / 16;
    a.G = lmhead_grid_x(M, V);
    const dim3 grid(a.G, lmhead_grid_y(M));
    switch (row_tiles_per_chunk(M)) {
        case 1: return launch_mt<1>(a, grid, s);
        case 2: return launch_mt<2>(a, grid, s);
        case 3: return launch_mt<3>(a, grid, s);
        case 4: return launch_mt<4>(a, grid, s);
        case 5: return launch_mt<5>(a, grid, s);
        case 6: return launch_mt<6>(a, grid, s);
        case 7: return launch_mt<7>(a, grid, s);
        case 8: return launch_mt<8>(a, grid, s);
        case 9: return launch_mt<9>(a, grid, s);
        case 10: return launch_mt<10>(a, grid, s);
        case 11: return launch_mt<11>(a, grid, s);
        case 12: return launch_mt<12>(a, grid, s);
        case 13: return launch_mt<13>(a, grid, s);
        case 14: return launch_mt<14>(a, grid, s);
        case 15: return launch_mt<15>(a, grid, s);
        default: return launch_mt<16>(a, grid, s);
    }
}

hipError_t launch_lse_combine(const float2* lse_part, int nparts, float* lse, int M, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(lse_combine_kernel, dim3(M), dim3(64), 0, s, lse_part, nparts, lse, M);
    return hipGetLastError();
}

hipError_t launch_row_lse(const float* logits, int64_t ldz, float* lse, int M, int V, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(row_lse_kernel, dim3(M), dim3(256), 0, s, logits, ldz, lse, V);
    return hipGetLastError();
}

}  // namespace dflash
