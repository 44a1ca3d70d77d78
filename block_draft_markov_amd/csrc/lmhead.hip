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

#include <type_traits>

namespace dflash {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;                       // h elements per stage
constexpr int kRowBytes = kBK * 2 + 16;       // padded LDS row: conflict-free 16-byte reads
constexpr int kNT = 4;      // vocab tiles per wave per pass of the small-row kernel
constexpr int kDepth = 4;   // its W register ring

struct LmHeadArgs {
    const uint16_t* hidden;
    const uint16_t* W;
    float* logits;
    float2* part;
    int64_t ldz;
    int M, H, V;
    int tiles;   // vocab tiles: ceil(V / 16) for the small-row kernel, ceil(V / 32) for the batched one
    int G;       // workgroups along the vocabulary
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_impl<I + 1, N>(f);
    }
}
// f(integral_constant<0>) ... f(integral_constant<N-1>), unrolled at compile time
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, N>(f); }

constexpr int gcd_c(int x, int y) { return y == 0 ? x : gcd_c(y, x % y); }
constexpr int lcm3(int x, int y, int z) {
    return (x / gcd_c(x, y) * y) / gcd_c(x / gcd_c(x, y) * y, z) * z;
}

__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
    if (s2 == 0.f) return;
    if (s == 0.f) { m = m2; s = s2; return; }
    float mn = fmaxf(m, m2);
    s = s * expf(m - mn) + s2 * expf(m2 - mn);
    m = mn;
}

template <int MT, int NT, int DEPTH>
__global__ void __launch_bounds__(kThreads) lmhead_gemm_lse_kernel(LmHeadArgs a) {
    constexpr int ROWS = MT * 16;
    constexpr int CHUNKS = ROWS * (kBK / 8);                  // 16-byte pieces of a hidden stage
    constexpr int PER_THREAD = (CHUNKS + kThreads - 1) / kThreads;
    // one spare row takes the writes of the surplus threads of the last hidden
    // chunk round, so that stores need no branch
    __shared__ __attribute__((aligned(16))) uint8_t hs[2][ROWS + 1][kRowBytes];
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

    // hidden stage ks -> registers.  Loads are never skipped or masked at load
    // time: an out-of-range piece loads a clamped, valid address and is zeroed
    // when it is written to LDS.  (A branch or a select right after a load makes
    // the compiler wait for that load at once, which would serialise the pipeline.)
    auto load_h = [&](int ks, bf16x8 (&reg)[PER_THREAD]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int c = tid + i * kThreads;
            const int row = c >> 3, col = ks * kBK + (c & 7) * 8;
            const int grow = min(m0 + row, a.M - 1), gcol = min(col, H - 8);
            reg[i] = *reinterpret_cast<const bf16x8*>(a.hidden + (int64_t)grow * H + gcol);
        }
    };
    auto store_h = [&](int buf, int ks, const bf16x8 (&reg)[PER_THREAD]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
            const int c = tid + i * kThreads;
            const int row = c >> 3, col = ks * kBK + (c & 7) * 8;
            const bool ok = c < CHUNKS && m0 + row < a.M && col < H;
            *reinterpret_cast<bf16x8*>(&hs[buf][min(row, ROWS)][(c & 7) * 16]) = ok ? reg[i] : bf16x8{};
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
        auto load_w = [&](int ks, bf16x8 (&w)[NT][2]) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const int col = ks * kBK + lg * 16 + s * 8;
                    // columns past H meet zeroed hidden values; rows of invalid tiles are dropped
                    w[j][s] = __builtin_nontemporal_load(wrow[j] + (min(col, H - 8) >> 3));
                }
            }
        };

        f32x4 acc[MT][NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        // Software pipeline over 64-wide h steps.  W(s) is loaded at step s-(DEPTH-1) into
        // wbuf[s % DEPTH]; hidden(s) is loaded at step s-2 into hreg[s % 2] and written to
        // LDS buffer s % 2 at the end of step s-1.  Every W load is issued after the hidden
        // load that the next LDS write waits for, so that wait never forces a young W load.
        bf16x8 hreg[2][PER_THREAD];
        bf16x8 wbuf[DEPTH][NT][2];
        load_h(0, hreg[0]);
        load_h(1, hreg[1]);
#pragma unroll
        for (int d = 0; d < DEPTH - 1; ++d) load_w(d, wbuf[d]);
        store_h(0, 0, hreg[0]);
        __syncthreads();

        // one 64-wide step: prefetch hidden(ks+2) and W(ks+DEPTH-1), multiply step ks,
        // write hidden(ks+1) to LDS.  In the main loop nothing is conditional
        // (prefetches past the end read clamped addresses and are never used), so
        // the compiler can count outstanding loads exactly.
        auto step = [&](auto U, int ks) __attribute__((always_inline)) {
            constexpr int u = decltype(U)::value;
            load_h(ks + 2, hreg[u & 1]);
            load_w(ks + DEPTH - 1, wbuf[(u + DEPTH - 1) % DEPTH]);
            // the B fragments of row tile mt+1 are read from LDS while tile mt multiplies
            const uint8_t* base = &hs[u & 1][lr][lg * 32];
            bf16x8 hb[2][2];
            hb[0][0] = *reinterpret_cast<const bf16x8*>(base);
            hb[0][1] = *reinterpret_cast<const bf16x8*>(base + 16);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mt + 1 < MT) {
                    const uint8_t* rowp = base + (mt + 1) * 16 * kRowBytes;
                    hb[(mt + 1) & 1][0] = *reinterpret_cast<const bf16x8*>(rowp);
                    hb[(mt + 1) & 1][1] = *reinterpret_cast<const bf16x8*>(rowp + 16);
                }
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wbuf[u % DEPTH][j][0], hb[mt & 1][0], acc[mt][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[mt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wbuf[u % DEPTH][j][1], hb[mt & 1][1], acc[mt][j], 0, 0, 0);
            }
            store_h((u + 1) & 1, ks + 1, hreg[(u + 1) & 1]);
            __syncthreads();
        };
        // UN steps per iteration keep every ring slot a compile-time register choice
        constexpr int UN = (DEPTH % 2 == 0) ? DEPTH : 2 * DEPTH;
        const int nmain = nks - nks % UN;
        for (int ks0 = 0; ks0 < nmain; ks0 += UN) {
            static_for<UN>([&](auto U) __attribute__((always_inline)) { step(U, ks0 + decltype(U)::value); });
        }
        // the remaining steps use the same slots, since nmain is a multiple of UN
        static_for<UN - 1>([&](auto U) __attribute__((always_inline)) {
            if (nmain + decltype(U)::value < nks) step(U, nmain + decltype(U)::value);
        });

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
                    if (tvalid[j] && v0 + q < a.V) sm += __expf(acc[mt][j][q] - mx);
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

// ---------------------------------------------------------------- batched row tiles
// More than 64 rows: a warp-specialised kernel.  Of the 8 waves of a
// workgroup, waves 4..7 are producers: they only move data, W rows of the
// pass and the hidden rows of the batch, from HBM and L2 into a 3-slot LDS
// ring, through a register ring that keeps loads STEP_AHEAD 64-wide steps in
// flight.  Waves 0..3 are consumers: they only read MFMA operands from LDS
// and issue v_mfma_f32_32x32x16_bf16 (on gfx950 it sustains about 2.2
// PFLOP/s with two accumulator chains; the 16x16x32 form reaches barely
// half).  A producer's wait for its loads therefore never stalls an MFMA,
// and memory and matrix work overlap instead of adding up.
// Consumer w owns vocab tile w (32 rows) of every pass and all MT 32-row
// tiles of the batch.  Operands: lane l covers row l % 32 and, in sub-step s
// of a 64-wide step, reduction indices 64 ks + 32 (l / 32) + 8 s .. +7, the
// same in A (W) and B (hidden).  Result register r of lane l is vocab entry
// 8 (r / 4) + 4 (l / 32) + r % 4 of the tile for batch row l % 32, so a lane
// stores four runs of four consecutive logits.
// LDS rows are 128 bytes with the 16-byte chunk c of row r kept at chunk
// c ^ swz(r), which makes the fragment reads conflict-free for 32- and
// 64-bank LDS without padding.
constexpr int kPcThreads = 512;
constexpr int kConsumers = 4;
constexpr int kSlots = 3;
constexpr int kStepAhead = 3;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <int MT>
__global__ void __launch_bounds__(kPcThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
lmhead_pc_kernel(LmHeadArgs a) {
    constexpr int BN = kConsumers * 32;              // vocab rows per pass
    constexpr int HR = MT * 32;                      // batch rows staged
    constexpr int WP = BN * 8 / 256;                 // W pieces per producer thread per step
    constexpr int HP = (HR * 8 + 255) / 256;         // hidden pieces per producer thread per step
    __shared__ __attribute__((aligned(16))) uint8_t wsm[kSlots][BN][128];
    __shared__ __attribute__((aligned(16))) uint8_t hsm[kSlots][HR][128];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int b = blockIdx.x;
    const int m0 = blockIdx.y * HR;                  // first batch row of this row chunk
    const int t_begin = (int)((int64_t)b * a.tiles / a.G);
    const int t_end = (int)((int64_t)(b + 1) * a.tiles / a.G);
    const int H = a.H;
    const int nks = (H + kBK - 1) / kBK;
    const int hchunks = H / 8;

    // Both roles walk the same passes and steps, with one barrier per step plus one per pass,
    // so their __syncthreads calls pair up.
    if (wave >= kConsumers) {
        // ================= producers: HBM / L2 -> registers -> LDS ring
        const int ptid = tid - kConsumers * 64;      // 0..255
        const int pc = ptid & 7;                     // 16-byte chunk of the pieces of this thread
        const uint16_t* hsrc[HP];
#pragma unroll
        for (int q = 0; q < HP; ++q) {
            const int row = (ptid + 256 * q) >> 3;
            hsrc[q] = a.hidden + (int64_t)min(m0 + row, a.M - 1) * H;
        }
        for (int pt = t_begin; pt < t_end; pt += kConsumers) {
            const bf16x8* wsrc[WP];
#pragma unroll
            for (int q = 0; q < WP; ++q) {
                const int v = min(pt * 32 + ((ptid + 256 * q) >> 3), a.V - 1);
                wsrc[q] = reinterpret_cast<const bf16x8*>(a.W + (int64_t)v * H);
            }
            auto load_step = [&](int ks, bf16x8 (&rw)[WP], bf16x8 (&rh)[HP]) __attribute__((always_inline)) {
                const int chunk = min(ks * 8 + pc, hchunks - 1);
#pragma unroll
                for (int q = 0; q < WP; ++q) rw[q] = __builtin_nontemporal_load(wsrc[q] + chunk);
#pragma unroll
                for (int q = 0; q < HP; ++q) rh[q] = *reinterpret_cast<const bf16x8*>(hsrc[q] + chunk * 8);
            };
            auto store_step = [&](int slot, int ks, const bf16x8 (&rw)[WP], const bf16x8 (&rh)[HP])
                __attribute__((always_inline)) {
                const bool colok = ks * kBK + pc * 8 < H;    // columns past H are zero
#pragma unroll
                for (int q = 0; q < WP; ++q) {
                    const int row = (ptid + 256 * q) >> 3;
                    *reinterpret_cast<bf16x8*>(&wsm[slot][row][(pc ^ swz(row)) * 16]) = colok ? rw[q] : bf16x8{};
                }
#pragma unroll
                for (int q = 0; q < HP; ++q) {
                    const int row = (ptid + 256 * q) >> 3;
                    const bool ok = colok && m0 + row < a.M;
                    *reinterpret_cast<bf16x8*>(&hsm[slot][row][(pc ^ swz(row)) * 16]) = ok ? rh[q] : bf16x8{};
                }
            };
            bf16x8 rw[kStepAhead][WP], rh[kStepAhead][HP];
            // prologue: steps 0 .. kStepAhead-1 in flight, step 0 written to slot 0
            static_for<kStepAhead>([&](auto D) __attribute__((always_inline)) {
                load_step(decltype(D)::value, rw[decltype(D)::value], rh[decltype(D)::value]);
            });
            store_step(0, 0, rw[0], rh[0]);
            __syncthreads();
            // step ks: refill ring entry ks % kStepAhead with step ks + kStepAhead, then write
            // step ks + 1 (loaded kStepAhead - 1 steps ago) into slot (ks + 1) % kSlots
            auto pstep = [&](auto U, int ks) __attribute__((always_inline)) {
                constexpr int u = decltype(U)::value;
                load_step(ks + kStepAhead, rw[u % kStepAhead], rh[u % kStepAhead]);
                store_step((u + 1) % kSlots, ks + 1, rw[(u + 1) % kStepAhead], rh[(u + 1) % kStepAhead]);
                __syncthreads();
            };
            constexpr int UN = lcm3(kStepAhead, kSlots, 1);
            const int nmain = nks - nks % UN;
            for (int ks0 = 0; ks0 < nmain; ks0 += UN)
                static_for<UN>([&](auto U) __attribute__((always_inline)) { pstep(U, ks0 + decltype(U)::value); });
            static_for<UN - 1>([&](auto U) __attribute__((always_inline)) {
                if (nmain + decltype(U)::value < nks) pstep(U, nmain + decltype(U)::value);
            });
        }
    } else {
        // ================= consumers: LDS -> MFMA, then the pass epilogue
        float run_m[MT], run_s[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) { run_m[i] = 0.f; run_s[i] = 0.f; }
        for (int pt = t_begin; pt < t_end; pt += kConsumers) {
            const int tile = pt + wave;                  // this wave's vocab tile
            const bool cvalid = tile < t_end;
            f32x16 acc[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[i] = f32x16{};
            __syncthreads();   // pairs with the producers' prologue barrier
            auto cstep = [&](auto U, int ks) __attribute__((always_inline)) {
                constexpr int slot = decltype(U)::value % kSlots;
                if (cvalid) {
                    bf16x8 af[4];
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int r = wave * 32 + lr;
                        af[s] = *reinterpret_cast<const bf16x8*>(&wsm[slot][r][((4 * lh + s) ^ swz(r)) * 16]);
                    }
#pragma unroll
                    for (int i = 0; i < MT; ++i) {
                        const int r = i * 32 + lr;
                        bf16x8 hb[4];
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            hb[s] = *reinterpret_cast<const bf16x8*>(&hsm[slot][r][((4 * lh + s) ^ swz(r)) * 16]);
#pragma unroll
                        for (int s = 0; s < 4; ++s)
                            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s], hb[s], acc[i], 0, 0, 0);
                    }
                }
                __syncthreads();
            };
            constexpr int UN = kSlots;
            const int nmain = nks - nks % UN;
            for (int ks0 = 0; ks0 < nmain; ks0 += UN)
                static_for<UN>([&](auto U) __attribute__((always_inline)) { cstep(U, ks0 + decltype(U)::value); });
            static_for<UN - 1>([&](auto U) __attribute__((always_inline)) {
                if (nmain + decltype(U)::value < nks) cstep(U, nmain + decltype(U)::value);
            });

            // ---- epilogue of the pass: logits and the rows' (max, sum exp) over this tile
            if (cvalid) {
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int m = m0 + i * 32 + lr;
                    float mx = -INFINITY;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int v0 = tile * 32 + 8 * g + 4 * lh;
                        const f32x4 z = {acc[i][4 * g], acc[i][4 * g + 1], acc[i][4 * g + 2], acc[i][4 * g + 3]};
                        if (m < a.M) {
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
                            if (v0 + q < a.V) mx = fmaxf(mx, z[q]);
                    }
                    float sm = 0.f;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int v0 = tile * 32 + 8 * g + 4 * lh;
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (v0 + q < a.V) sm += __expf(acc[i][4 * g + q] - mx);
                    }
                    const float m2 = __shfl_xor(mx, 32);
                    const float s2 = __shfl_xor(sm, 32);
                    lse_merge(mx, sm, m2, s2);
                    lse_merge(run_m[i], run_s[i], mx, sm);
                }
            }
        }
        // one partial per (row, consumer wave): column b * kConsumers + wave of the partial array
        if (lh == 0) {
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int m = m0 + i * 32 + lr;
                if (m < a.M)
                    a.part[(int64_t)m * a.G * kConsumers + b * kConsumers + wave] = make_float2(run_m[i], run_s[i]);
            }
        }
    }
}

template <int MT>
hipError_t launch_mt(const LmHeadArgs& a, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((lmhead_gemm_lse_kernel<MT, kNT, kDepth>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_pc(const LmHeadArgs& a, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((lmhead_pc_kernel<MT>), grid, dim3(kPcThreads), 0, s, a);
    return hipGetLastError();
}

// Up to 64 rows: the vocab-split kernel with ceil(M / 16) row tiles.  More:
// the warp-specialised kernel on row chunks of up to 224 rows (seven 32-row
// tiles: the most whose accumulators and load rings fit the register file).
constexpr int kPcMaxRows = 224;
bool small_rows(int M) { return M <= 64; }
int row_tiles_small(int M) { return M <= 0 ? 1 : (M + 15) / 16; }
int pc_chunks(int M) { return (M + kPcMaxRows - 1) / kPcMaxRows; }
int pc_tiles(int M) {   // 32-row tiles per chunk
    const int gy = pc_chunks(M);
    return ((M + gy - 1) / gy + 31) / 32;
}
// workgroups along the vocabulary
int lmhead_grid(int M, int V) {
    if (small_rows(M)) {
        const int tiles = (V + 15) / 16;
        const int need = (tiles + 4 * kNT - 1) / (4 * kNT);
        const int cap = row_tiles_small(M) <= 2 ? 1024 : 512;
        return need < cap ? need : cap;
    }
    const int tiles = (V + 31) / 32;
    const int need = (tiles + kConsumers - 1) / kConsumers;
    const int cap = 256 / pc_chunks(M) > 0 ? 256 / pc_chunks(M) : 1;
    return need < cap ? need : cap;
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

int lmhead_partials(int M, int V) {
    return small_rows(M) ? lmhead_grid(M, V) : lmhead_grid(M, V) * kConsumers;
}

hipError_t launch_lmhead(const uint16_t* hidden, const uint16_t* W, float* logits, int64_t ldz,
                         float2* lse_part, int M, int H, int V, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    LmHeadArgs a;
    a.hidden = hidden; a.W = W; a.logits = logits; a.part = lse_part; a.ldz = ldz;
    a.M = M; a.H = H; a.V = V;
    a.G = lmhead_grid(M, V);
    if (small_rows(M)) {
        a.tiles = (V + 15) / 16;
        const dim3 grid(a.G, 1);
        switch (row_tiles_small(M)) {
            case 1: return launch_mt<1>(a, grid, s);
            case 2: return launch_mt<2>(a, grid, s);
            case 3: return launch_mt<3>(a, grid, s);
            default: return launch_mt<4>(a, grid, s);
        }
    }
    a.tiles = (V + 31) / 32;
    const dim3 grid(a.G, pc_chunks(M));
    switch (pc_tiles(M)) {
        case 3: return launch_pc<3>(a, grid, s);
        case 4: return launch_pc<4>(a, grid, s);
        case 5: return launch_pc<5>(a, grid, s);
        case 6: return launch_pc<6>(a, grid, s);
        default: return launch_pc<7>(a, grid, s);
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
