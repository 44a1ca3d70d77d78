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
// One launch per position (the next position needs every request's choice).  A
// workgroup takes kIds vocabulary ids (kTpw tiles of 32 per wave) for up to kGroup
// requests; the biases are a small fp32 GEMM (ids x requests x rank) on the matrix
// cores, fed by B rows streamed through registers a 128-byte line at a time and the
// requests' A rows staged in LDS.  Per request the largest x with the lowest id is
// packed into one 64-bit entry (order-preserving key of x << 32 | ~id); one atomicMax
// per request and workgroup merges the workgroups.  The kernel is bound by the B
// stream: V_d r 4 bytes per position, every position.

#include "common.hpp"
#include "internal.hpp"

#include <math.h>

namespace dflash {

namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 32;     // requests per workgroup
constexpr int kBufWord3 = 0x00020000;   // gfx9 buffer descriptor word 3: raw dword access
constexpr int kBig = 0x40000000;        // buffer offset past the end of every table the buffer path takes
constexpr int kRankChunk = 256; // rank elements of the A rows staged in LDS at a time
constexpr int kAhead = 1;   // 32-element slots of B in flight ahead of the MFMAs
constexpr int kTpw = 3;     // 32-id vocab tiles per wave (one, two and four measured slower)
constexpr int kIds = 4 * 32 * kTpw;   // vocab ids per workgroup
constexpr int kAStride = kRankChunk + 4;   // padded row stride: the 32 rows of a read hit distinct banks

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

// One position for kGroup (32) requests and kIds vocabulary ids: wave w computes the
// bias of kTpw tiles of 32 ids for the 32 requests with v_mfma_f32_32x32x2_f32 (fp32
// products and sums), the B rows of the ids as the row operand and the A rows of the
// requests' previous tokens (staged in LDS) as the column operand.  In MFMA step s lane l
// supplies B[t(id l % 32)][k] and A[s(request l % 32)][k] with k = 8 (s / 4) + 4 (l / 32)
// + s % 4, the same index in both, so a lane reads 4 consecutive rank elements per 4
// steps.  Result register i of lane l is id 8 (i / 4) + 4 (l / 32) + i % 4 of the tile
// for request l % 32: a lane holds 16 ids of one request, so the argmax is taken in
// the lane and finished with one exchange between the two halves of the wave.
template <bool kVec>
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

    // the B rows of this lane's vocab ids in the wave's tiles
    const int vt0 = blockIdx.x * kIds + w * 32 * kTpw;   // first id of the wave's tiles
    const float* brow[kTpw];
    bool bok[kTpw];
#pragma unroll
    for (int j = 0; j < kTpw; ++j) {
        const int v = vt0 + 32 * j + lr;
        bok[j] = v < V;
        int64_t t = bok[j] ? target_of(v, d2t) : 0;
        t = t < 0 ? 0 : (t >= Vt ? (int64_t)Vt - 1 : t);
        brow[j] = TB + t * r;
    }
    // Loads without branches or selects (either makes the wave wait for the load at once,
    // which would leave one group in flight).  kVec: buffer loads of 16 bytes whose offset
    // is moved past the end of the table for lanes past the rank or the vocabulary, where
    // the hardware returns zeros.  Otherwise (a rank that is not a multiple of 4, or a
    // table of 2^30 bytes or more) scalar loads from clamped addresses and selects.
    const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(TB), (short)0, (int)min((int64_t)Vt * r * 4, (int64_t)kBig), kBufWord3);
    int boff[kTpw];
    if constexpr (kVec) {
#pragma unroll
        for (int j = 0; j < kTpw; ++j) boff[j] = bok[j] ? (int)((brow[j] - TB) * 4) : kBig;
    }
    auto load_b = [&](int k0, int j) __attribute__((always_inline)) -> f32x4 {
        const int k = k0 + 4 * lh;
        f32x4 x;
        if constexpr (kVec) {
            const int off = k < r ? boff[j] + 4 * k : kBig;
            x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(brsrc, off, 0, 0));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float raw = brow[j][min(k + e, r - 1)];
                x[e] = (bok[j] && k + e < r) ? raw : 0.f;
            }
        }
        return x;
    };
    // B runs kAhead slots ahead of the MFMAs.  A slot is 32 rank elements, the whole
    // 128-byte line of every row: the 4 loads of a line leave back to back, so the line
    // moves from L2 once (loads of one line spread over time would each fetch it again
    // once L1 has dropped it).  Slot d of the ring holds elements kc + 32 d ..; each slot
    // is consumed, then refilled with the slot kAhead later (the last refills of a chunk
    // fetch the first slots of the next), so the loop carries the ring in place (a
    // register copy of a pending load would wait for it).  The first slots are requested
    // before anything else: they depend on nothing the setup reads.
    static_assert(kRankChunk % (32 * kAhead) == 0, "the ring depth divides the rank chunk");
    f32x4 ring[kAhead][kTpw][4];
#pragma unroll
    for (int d = 0; d < kAhead; ++d)
#pragma unroll
        for (int j = 0; j < kTpw; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) ring[d][j][t] = load_b(32 * d + 8 * t, j);

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
    // the logits of the epilogue (row of request lr, ids 8 c + 4 lh .. + 3 of every tile),
    // loaded now so that they arrive while the MFMAs run; the addresses are clamped into
    // the buffer and lanes without a valid (row, id) are masked in the epilogue
    const int myrow = mrow[lr];
    f32x4 zpre[kTpw][4];
    {
        const float* zr = logits + (int64_t)max(myrow, 0) * ldz;
#pragma unroll
        for (int j = 0; j < kTpw; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int id4 = min(vt0 + 32 * j + 8 * c + 4 * lh, (int)ldz - 4);
                zpre[j][c] = *reinterpret_cast<const f32x4*>(zr + id4);
            }
    }

    f32x16 acc[kTpw];
#pragma unroll
    for (int j = 0; j < kTpw; ++j) acc[j] = f32x16{};
    for (int c0 = 0; c0 < r; c0 += kRankChunk) {
        const int cn = min(kRankChunk, r - c0);
        const int cpad = (cn + 31) / 32 * 32;   // <= kRankChunk, a multiple of the 32-element slot
        __syncthreads();   // the previous chunk's reads are done
        if (kVec && cn == kRankChunk) {
            // a whole chunk: every thread issues its 8 loads of 16 bytes at once
            constexpr int kPer = kGroup * kRankChunk / 4 / kThreads;
            f32x4 av[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = tid + kThreads * i, q = e / (kRankChunk / 4), c4 = e % (kRankChunk / 4);
                av[i] = *reinterpret_cast<const f32x4*>(TA + arow[q] + c0 + 4 * c4);
            }
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int e = tid + kThreads * i, q = e / (kRankChunk / 4), c4 = e % (kRankChunk / 4);
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<f32x4*>(&As[q * kAStride + 4 * c4]) = mrow[q] >= 0 ? av[i] : zero;
            }
        } else {
            for (int e = tid; e < kGroup * cpad; e += kThreads) {
                const int q = e / cpad, i = e % cpad;
                As[q * kAStride + i] = (mrow[q] >= 0 && i < cn) ? TA[arow[q] + c0 + i] : 0.f;
            }
        }
        __syncthreads();
        // the A operand is read from LDS one 8-element group ahead (groups alternate
        // between avr[0] and avr[1]; a slot holds 4 groups, so the loop carries avr[0])
        const float* arow_lds = &As[lr * kAStride + 4 * lh];
        f32x4 avr[2];
        avr[0] = *reinterpret_cast<const f32x4*>(arow_lds);
        for (int kc = 0; kc < cpad; kc += 32 * kAhead) {
#pragma unroll
            for (int d = 0; d < kAhead; ++d) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    // the next 8-element group of A (past the chunk's end: a valid LDS
                    // address, value unused); groups alternate between avr[0] and avr[1]
                    avr[(t + 1) & 1] =
                        *reinterpret_cast<const f32x4*>(arow_lds + min(kc + 32 * d + 8 * (t + 1), cpad - 8));
                    __builtin_amdgcn_sched_barrier(0);   // issued before this group's MFMAs
                    const f32x4 av = avr[t & 1];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int j = 0; j < kTpw; ++j)
                            acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(ring[d][j][t][e], av[e], acc[j], 0, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < kTpw; ++j)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        ring[d][j][t] = load_b(c0 + kc + 32 * (d + kAhead) + 8 * t, j);
                __builtin_amdgcn_sched_barrier(0);   // keep the refill here, not clustered at the end
            }
        }
    }

    // x = f(z) + bias of request lr at the lane's ids, ascending (tile j, register i); the
    // lane keeps the largest x and, on a tie, the first (lowest) id
    const HeadMap hm = head_map(scale, cap);
    float bx = -INFINITY;
    uint32_t bid = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < kTpw; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int v = vt0 + 32 * j + 8 * (i / 4) + 4 * lh + i % 4;
            const float x = head_apply(hm, zpre[j][i / 4][i % 4]) + acc[j][i];
            if (v < V && x > bx) {
                bx = x;
                bid = (uint32_t)v;
            }
        }
    // the two halves hold interleaved ids of the same request: keep the larger x, the
    // lower id on a tie
    const float ox = __shfl_xor(bx, 32);
    const uint32_t oid = (uint32_t)__shfl_xor((int)bid, 32);
    if (ox > bx || (ox == bx && oid < bid)) {
        bx = ox;
        bid = oid;
    }
    if (lh == 0) wbest[w][lr] = (myrow >= 0 && bid != 0xFFFFFFFFu) ? pack_entry(float_to_key(bx), bid) : 0ull;
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
    const dim3 grid((V + kIds - 1) / kIds, (R + kGroup - 1) / kGroup);
    // the buffer path: 16-byte rows and a B table below 2^30 bytes (offsets stay below kBig)
    const bool vec = (r & 3) == 0 && (reinterpret_cast<uintptr_t>(tables) & 15) == 0 &&
                     (int64_t)Vt * r * 4 < (int64_t)kBig;
    for (int p = 0; p < L; ++p) {
        if (vec)
            hipLaunchKernelGGL(dense_pos_kernel<true>, grid, dim3(kThreads), 0, s, logits, ldz, d2t, tables,
                               last_tok, row_offsets, R, L, M, V, Vt, r, scale, cap, p, best);
        else
            hipLaunchKernelGGL(dense_pos_kernel<false>, grid, dim3(kThreads), 0, s, logits, ldz, d2t, tables,
                               last_tok, row_offsets, R, L, M, V, Vt, r, scale, cap, p, best);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(dense_finish_kernel, dim3((nb + kThreads - 1) / kThreads), dim3(kThreads), 0, s, best, d2t,
                       row_offsets, R, L, M, V, tokens, values);
    return hipGetLastError();
}

}  // namespace dflash
