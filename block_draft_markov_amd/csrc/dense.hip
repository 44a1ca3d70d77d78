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
// One launch per position (the next position needs every request's choice).  The
// biases are a small fp32 GEMM (ids x requests x rank) on the matrix cores; per request
// the largest x with the lowest id is packed into one 64-bit entry (order-preserving key
// of x << 32 | ~id), and one atomicMax per request and workgroup merges the workgroups.
// Two kernels compute a position:
//   - dense_lds_kernel (ranks that are a multiple of 4, up to 512): every operand byte is
//     staged in LDS by loads that write LDS directly, twelve waves per CU;
//   - dense_reg_kernel (every other rank): B rows streamed through registers a 128-byte
//     line at a time, the requests' A rows staged in LDS by rank chunks.
// Both are bound by the B stream: V_d r 4 bytes per position, every position.

#include "common.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

#include <math.h>

#include <algorithm>

namespace dflash {

namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 32;     // requests per workgroup
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

// Row of request req at position p, -1 when its block is shorter.
__device__ __forceinline__ int request_row(const int32_t* row_offsets, int req, int L, int M, int p) {
    int a, n;
    rows_of(row_offsets, req, L, M, a, n);
    return p < n ? a + p : -1;
}

// The previous token s_p of request req as a clamped target-vocabulary row: the last
// accepted token at p = 0, else t of the id the previous position chose.
__device__ __forceinline__ int64_t request_prev(const int64_t* last_tok, const uint64_t* best, const int64_t* d2t,
                                                int R, int V, int Vt, int p, int req) {
    int64_t s;
    if (p == 0) {
        s = last_tok[req];
    } else {
        const uint64_t e = best[(int64_t)(p - 1) * R + req];
        s = target_of(min((int64_t)entry_id(e), (int64_t)V - 1), d2t);
    }
    return s < 0 ? 0 : (s >= Vt ? (int64_t)Vt - 1 : s);
}

// Both of the above (m = -1 and s = 0 for a request without a row at p).
__device__ __forceinline__ void request_state(const int32_t* row_offsets, const int64_t* last_tok,
                                              const uint64_t* best, const int64_t* d2t, int R, int L, int M,
                                              int V, int Vt, int p, int req, int& m, int64_t& s) {
    m = request_row(row_offsets, req, L, M, p);
    s = m >= 0 ? request_prev(last_tok, best, d2t, R, V, Vt, p, req) : 0;
}

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
__global__ void __launch_bounds__(kThreads) dense_reg_kernel(
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
        if (tid < ng) request_state(row_offsets, last_tok, best, d2t, R, L, M, V, Vt, p, g0 + tid, m, s);
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

// ---------------------------------------------------------------- LDS-staged kernel
// The same position step for ranks that are a multiple of 4 up to kRankCapMax, with every
// table and the logits below 2^29 bytes.  Every operand byte moves with buffer_load ...
// lds into 4 KB slots of 32 rows of one 128-byte line (chunk c of row q at chunk
// c ^ swz(q)), so whole lines leave together and nothing passes through registers on
// its way in:
//   - the requests' A rows, all of the rank, loaded once and shared by the waves;
//   - per vocabulary tile, the r / 32 lines of its 32 B rows, then one line of the
//     requests' logits at the tile's ids.
// One workgroup per CU takes a contiguous range of tiles; its WPW waves take tiles t0 + w,
// t0 + w + WPW, ... and stream their slots through rings of their own of NS slots, NS - 1
// in flight ahead of the slot they compute.  The stream holds nothing but these loads,
// so each wait is an exact vmcnt count.  A B slot is 16 MFMAs (v_mfma_f32_32x32x2_f32,
// the operand layout of the register-streamed kernel above) on two accumulators, even
// and odd steps; the logits slot closes the tile: x = f(z) + both accumulators, and the
// lane keeps its best.  The kernel is bound by the B stream.
constexpr int kSlot = 32 * 128;        // bytes of a slot: 32 rows of one 128-byte line
constexpr int kMaxWgTiles = 32;        // vocabulary tiles per workgroup (LDS table of B row offsets)
constexpr int kRankCapMax = 512;
constexpr int kCUs = 256;              // MI355X compute units
// Ring slots per wave and waves per workgroup (ranks up to 256, and up to 512): more waves
// per SIMD hide one wave's load waits behind another's MFMAs better than deeper rings do
// (measured at the Qwen3-4B batch: 4 waves with 3-7 slots 47-49 us per position, 8 waves
// with 2 slots 41 us, 12 waves with 2 slots 39 us).
constexpr int kNS256 = 2, kWPW256 = 12;
constexpr int kNS512 = 2, kWPW512 = 8;

struct DenseArgs {
    const float* logits;
    const int64_t* d2t;
    const float* tables;
    const int64_t* last_tok;
    const int32_t* row_offsets;
    uint64_t* best;
    int64_t ldz;
    int R, L, M, V, Vt, r, p;
    float scale, cap;
};

constexpr int kWaitLgkm0 = 0xC07F;   // s_waitcnt lgkmcnt(0), vmcnt and expcnt unconstrained

// s_waitcnt vmcnt(4 n): the loads of n slots may still be in flight (n < 8)
__device__ __forceinline__ void wait_slots(int n) {
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(4)); break;
        case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(8)); break;
        case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm(12)); break;
        case 4: __builtin_amdgcn_s_waitcnt(waitcnt_vm(16)); break;
        case 5: __builtin_amdgcn_s_waitcnt(waitcnt_vm(20)); break;
        case 6: __builtin_amdgcn_s_waitcnt(waitcnt_vm(24)); break;
        default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(28)); break;
    }
}

template <int RCAP, int NS, int WPW>
__global__ void __launch_bounds__(64 * WPW) __attribute__((amdgpu_waves_per_eu(WPW / 4, WPW / 4)))
dense_lds_kernel(DenseArgs a) {
    static_assert(NS >= 2 && NS <= 8, "ring depth");
    static_assert(WPW == 4 || WPW == 8 || WPW == 12, "one to three waves per SIMD");
    constexpr int kT = 64 * WPW;
    constexpr int kALines = RCAP / 32;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[(kALines + WPW * NS) * kSlot];
    __shared__ int boff[kMaxWgTiles * 32];   // byte offsets of the workgroup's B rows (kBig: past V)
    __shared__ int zrow[kGroup], arow[kGroup];   // byte offsets of the requests' logits and A rows
    __shared__ int mrow[kGroup];             // the request's row at position p, -1 when it has none
    __shared__ uint64_t wbest[WPW][kGroup];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lh = lane >> 5, lrow = lane >> 3;
    const int g0 = blockIdx.y * kGroup;
    const int ng = min(kGroup, a.R - g0);
    const int tiles = (a.V + 31) / 32;
    const int t0 = (int)((int64_t)blockIdx.x * tiles / gridDim.x);
    const int t1 = (int)((int64_t)(blockIdx.x + 1) * tiles / gridDim.x);
    const int nl = (a.r + 31) / 32;          // lines of a table row
    const int rb = a.r * 4;                  // bytes of a table row

    // the requests' rows at p and the B row offsets of the workgroup's ids: nothing here
    // depends on the previous position, so the first B slots leave before its result is read
    if (tid < kGroup) {
        const int m = tid < ng ? request_row(a.row_offsets, g0 + tid, a.L, a.M, a.p) : -1;
        mrow[tid] = m;
        zrow[tid] = m >= 0 ? (int)((int64_t)m * a.ldz * 4) : kBig;
    }
    for (int i = tid; i < (t1 - t0) * 32; i += kT) {
        const int v = t0 * 32 + i;
        int o = kBig;
        if (v < a.V) {
            int64_t t = target_of(v, a.d2t);
            t = t < 0 ? 0 : (t >= a.Vt ? (int64_t)a.Vt - 1 : t);
            o = (int)(t * rb);
        }
        boff[i] = o;
    }
    __syncthreads();

    const u32x4 tab_a = sbuf(a.tables, (int64_t)a.Vt * rb);
    const u32x4 tab_b = sbuf(a.tables + (int64_t)a.Vt * a.r, (int64_t)a.Vt * rb);
    const u32x4 zbuf = sbuf(a.logits, (int64_t)a.M * a.ldz * 4);
    // DMA instruction j of a slot fills rows 8 j + lane / 8; the lane fetches chunk gc[j]
    int gc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) gc[j] = (lane & 7) ^ swz(8 * j + lrow);
    // the wave's stream: ntw tiles of nl B slots and one logits slot each
    const int ntw = t1 - t0 > w ? (t1 - t0 - w + WPW - 1) / WPW : 0;
    const int S = ntw * (nl + 1);
    const uint32_t ring = lds0 + (kALines + w * NS) * kSlot;
    int zo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) zo[j] = zrow[8 * j + lrow];
    int bo[4];
    int in = 0, ij = 0, ipos = 0, issued = 0;   // issue cursor: tile, slot in the tile, ring slot
    auto issue = [&]() __attribute__((always_inline)) {
        const uint32_t dst = ring + ipos * kSlot;
        const int tl = w + WPW * in;               // tile within the workgroup's range
        if (ij == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) bo[j] = boff[tl * 32 + 8 * j + lrow];
        }
        if (ij < nl) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool ok = bo[j] != kBig && 32 * ij + 4 * gc[j] < a.r;
                dma16(tab_b, dst + j * 1024, ok ? bo[j] + 128 * ij + 16 * gc[j] : kBig, 0);
            }
        } else {
            const int col = 128 * (t0 + tl);
#pragma unroll
            for (int j = 0; j < 4; ++j) dma16(zbuf, dst + j * 1024, zo[j] != kBig ? zo[j] + col + 16 * gc[j] : kBig, 0);
        }
        ++issued;
        ipos = ipos == NS - 1 ? 0 : ipos + 1;
        if (++ij > nl) {
            ij = 0;
            ++in;
        }
    };
    const int pro = S < NS - 1 ? S : NS - 1;
    for (int i = 0; i < pro; ++i) issue();
    // the previous tokens and their A rows (loads complete in order: reading the previous
    // position's result also waits for the B slots issued above, which left first)
    if (tid < kGroup) {
        const int m = mrow[tid];
        arow[tid] = m >= 0 ? (int)(request_prev(a.last_tok, a.best, a.d2t, a.R, a.V, a.Vt, a.p, g0 + tid) * rb) : kBig;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // the A rows: instruction j of line c is issued by wave (4 c + j) % WPW
    for (int e = w; e < 4 * nl; e += WPW) {
        const int c = e >> 2, j = e & 3;
        const int ao = arow[8 * j + lrow];
        const int gcq = (lane & 7) ^ swz(8 * j + lrow);
        const bool ok = ao != kBig && 32 * c + 4 * gcq < a.r;
        dma16(tab_a, lds0 + c * kSlot + j * 1024, ok ? ao + 128 * c + 16 * gcq : kBig, 0);
    }

    // this wave's A lines, the last loads it issued, have landed; after the barrier every
    // wave's have
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // fragment byte offsets within a slot: row lr, chunk 2 c + lh
    int foff[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) foff[c] = lr * 128 + (((2 * c + lh) ^ swz(lr)) * 16);
    const HeadMap hm = head_map(a.scale, a.cap);
    float bx = -INFINITY;
    uint32_t bid = 0xFFFFFFFFu;
    int g = 0, cpos = 0;                         // compute cursor: stream slot, ring slot
    // the next slot of the stream has landed: returns its LDS bytes
    auto next_slot = [&]() __attribute__((always_inline)) -> const uint8_t* {
        if (issued < S) issue();
        wait_slots(issued - 1 - g);
        asm volatile("" ::: "memory");
        const uint8_t* sp = smem + (ring - lds0) + cpos * kSlot;
        ++g;
        cpos = cpos == NS - 1 ? 0 : cpos + 1;
        return sp;
    };
    for (int n = 0; n < ntw; ++n) {
        f32x16 acc0 = {}, acc1 = {};
        for (int c0 = 0; c0 < nl; ++c0) {
            const uint8_t* sp = next_slot();
            const uint8_t* ap = smem + c0 * kSlot;
            f32x4 bv[4], av[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                bv[c] = *reinterpret_cast<const f32x4*>(sp + foff[c]);
                av[c] = *reinterpret_cast<const f32x4*>(ap + foff[c]);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[c][0], av[c][0], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[c][1], av[c][1], acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[c][2], av[c][2], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[c][3], av[c][3], acc1, 0, 0, 0);
            }
        }
        // x of request lr at ids 8 (i / 4) + 4 lh + i % 4 of the tile, ascending; the lane
        // keeps the largest and, on a tie, the first (lowest) id
        const uint8_t* sp = next_slot();
        f32x4 zv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) zv[c] = *reinterpret_cast<const f32x4*>(sp + foff[c]);
        const int vb = 32 * (t0 + w + WPW * n) + 4 * lh;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int v = vb + 8 * (i / 4) + i % 4;
            const float x = head_apply(hm, zv[i / 4][i % 4]) + (acc0[i] + acc1[i]);
            if (v < a.V && x > bx) {
                bx = x;
                bid = (uint32_t)v;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

    // the two halves hold interleaved ids of the same request: keep the larger x, the
    // lower id on a tie
    const float ox = __shfl_xor(bx, 32);
    const uint32_t oid = (uint32_t)__shfl_xor((int)bid, 32);
    if (ox > bx || (ox == bx && oid < bid)) {
        bx = ox;
        bid = oid;
    }
    if (lh == 0) wbest[w][lr] = (mrow[lr] >= 0 && bid != 0xFFFFFFFFu) ? pack_entry(float_to_key(bx), bid) : 0ull;
    __syncthreads();
    if (tid < ng && mrow[tid] >= 0) {
        uint64_t bb = wbest[0][tid];
        for (int k = 1; k < WPW; ++k) bb = wbest[k][tid] > bb ? wbest[k][tid] : bb;
        atomicMax(reinterpret_cast<unsigned long long*>(&a.best[(int64_t)a.p * a.R + g0 + tid]),
                  (unsigned long long)bb);
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
    const int gy = (R + kGroup - 1) / kGroup;
    // the LDS-staged kernel: 16-byte table rows of at most kRankCapMax elements, tables and
    // logits within one buffer descriptor's range, 16-byte aligned logits rows
    const bool staged = (r & 3) == 0 && r <= kRankCapMax && (reinterpret_cast<uintptr_t>(tables) & 15) == 0 &&
                        (reinterpret_cast<uintptr_t>(logits) & 15) == 0 && (ldz & 3) == 0 &&
                        (int64_t)Vt * r * 4 < kDmaRange && (int64_t)M * ldz * 4 < kDmaRange;
    if (staged) {
        // one workgroup per CU (256) with at least four tiles, at most kMaxWgTiles tiles per
        // workgroup
        const int tiles = (V + 31) / 32;
        const int gx = std::max(std::min((tiles + 3) / 4, kCUs), (tiles + kMaxWgTiles - 1) / kMaxWgTiles);
        DenseArgs a{logits, d2t, tables, last_tok, row_offsets, best, ldz, R, L, M, V, Vt, r, 0, scale, cap};
        for (int p = 0; p < L; ++p) {
            a.p = p;
            if (r <= 256)
                hipLaunchKernelGGL((dense_lds_kernel<256, kNS256, kWPW256>), dim3(gx, gy), dim3(64 * kWPW256), 0, s, a);
            else
                hipLaunchKernelGGL((dense_lds_kernel<kRankCapMax, kNS512, kWPW512>), dim3(gx, gy), dim3(64 * kWPW512), 0,
                                   s, a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    } else {
        const dim3 grid((V + kIds - 1) / kIds, gy);
        // the buffer path: 16-byte rows and a B table below 2^30 bytes (offsets stay below kBig)
        const bool vec = (r & 3) == 0 && (reinterpret_cast<uintptr_t>(tables) & 15) == 0 &&
                         (int64_t)Vt * r * 4 < (int64_t)kBig;
        for (int p = 0; p < L; ++p) {
            if (vec)
                hipLaunchKernelGGL(dense_reg_kernel<true>, grid, dim3(kThreads), 0, s, logits, ldz, d2t, tables,
                                   last_tok, row_offsets, R, L, M, V, Vt, r, scale, cap, p, best);
            else
                hipLaunchKernelGGL(dense_reg_kernel<false>, grid, dim3(kThreads), 0, s, logits, ldz, d2t, tables,
                                   last_tok, row_offsets, R, L, M, V, Vt, r, scale, cap, p, best);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    hipLaunchKernelGGL(dense_finish_kernel, dim3((nb + kThreads - 1) / kThreads), dim3(kThreads), 0, s, best, d2t,
                       row_offsets, R, L, M, V, tokens, values);
    return hipGetLastError();
}

}  // namespace dflash
