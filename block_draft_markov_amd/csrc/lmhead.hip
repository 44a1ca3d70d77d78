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
// One kernel for every batch size: the vocabulary is cut into tiles of 32 rows,
// one workgroup per CU owns a contiguous tile range and all rows of its row
// chunk, and every operand byte is staged through LDS by buffer loads that write
// LDS directly (see the kernel's notes below).  Batches of up to 64 rows give
// each wave one vocab tile per pass (128 W rows per workgroup and step: the W
// stream then runs at about 5.7 TB/s); larger batches two, which halves the
// re-reads of their hidden states.

#include "common.hpp"
#include "internal.hpp"
#include "lds_dma.hpp"

#include <math.h>

#include <type_traits>

namespace dflash {

namespace {

constexpr int kBK = 64;                       // h elements per stage

struct LmHeadArgs {
    const uint16_t* hidden;
    const uint16_t* W;
    float* logits;
    float2* part;
    float* tmax;     // per-tile maxima [M][ldt] or null
    int64_t ldt;
    int64_t ldz;
    int M, H, V;
    int tiles;   // vocab tiles: ceil(V / 32)
    int G;       // workgroups along the vocabulary
    const float* tau;   // per-row lower bound of the K-th largest logit (filtered kernel only)
    uint8_t* tmask;     // [M][ldt]: groups of four logits written per tile (filtered kernel only)
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

// ---------------------------------------------------------------- the kernel
// Four waves, one per SIMD, so that each wave may hold up to 512 registers:
// wave w accumulates NV (1 or 2) vocab tiles of 32 rows for all MT 32-row batch
// tiles of its row chunk (NV MT 32x32 fp32 accumulators, in AGPRs), using
// v_mfma_f32_32x32x16_bf16 (on gfx950 it sustains about 2.2 PFLOP/s with two
// accumulator chains; the 16x16x32 form reaches barely half).
//
// Operands: lane l covers row l % 32 and, in sub-step s of a 64-wide step,
// reduction indices 64 ks + 32 (l / 32) + 8 s .. +7, the same in A (W) and B
// (hidden).  Result register r of lane l is vocab entry 8 (r / 4) + 4 (l / 32)
// + r % 4 of the tile for batch row l % 32, so a lane stores four runs of four
// consecutive logits.  LDS rows are 128 bytes with the 16-byte chunk c of row
// r kept at chunk c ^ swz(r): the fragment reads are conflict-free without
// padding.
//
// Every operand byte moves with buffer_load ... lds: each instruction fetches
// eight whole 128-byte lines (eight lanes per row) and lands lane l's 16 bytes
// at LDS byte 16 l of the instruction's 1 KB block; choosing which chunk of
// its row each lane fetches makes that block the swizzled layout.  Rows past
// the matrix, columns past H and the tiles a wave does not own in a short pass
// get an offset past the described buffer range, so they read as zeros and
// cost no memory traffic.
//
// LDS holds two hidden slots shared by the waves and three W slots per wave
// (W runs two steps ahead).  One barrier per step: each wave first waits
// until its own share of the hidden chunk of the step has landed.  The steps
// of all passes of a workgroup form one stream, so the loads of the next pass
// are in flight while a pass ends with its logits and (max, sum exp)
// epilogue.  A pass normally gives each wave two tiles; the last pass of a
// workgroup spreads what is left at one tile per wave when it can.
constexpr int kRowsWaves = 4;             // waves, and so (max, sum) partials, per workgroup

constexpr int kNV = 2;                    // vocab tiles per wave and pass (more than 64 rows)
constexpr int kWSlots = 3;                // W slots per wave: W runs kWSlots - 1 steps ahead
template <int MT, bool HFULL, int NVT, int SW = kWSlots, bool FILTER = false>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
lmhead_dma_kernel(LmHeadArgs a) {
    static_assert(SW >= 3, "the wait before each barrier assumes W is issued two or more steps ahead");
    constexpr int NV = NVT;
    constexpr int WJ = NV * 4;                   // W DMA instructions per wave and step
    constexpr int HR = MT * 32;                  // batch rows staged
    constexpr int WR = NV * 32;                  // W rows of one wave per pass
    constexpr int HSLOT = HR * 128;              // bytes of a hidden slot
    constexpr int WSLOT = 4 * WR * 128;          // bytes of a W slot (all four waves)
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * HSLOT + SW * WSLOT];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31, lh = lane >> 5;
    const int b = blockIdx.x;
    const int m0 = blockIdx.y * HR;
    const int t_begin = (int)((int64_t)b * a.tiles / a.G);
    const int t_end = (int)((int64_t)(b + 1) * a.tiles / a.G);
    const int H = a.H;
    const int nks = (H + kBK - 1) / kBK;
    const int hchunks = H / 8;

    // pass plan: nfull passes of 4 NV tiles, then one pass over the rest (one tile per wave when it fits)
    const int T = t_end - t_begin;
    const int nfull = T / (4 * NV);
    const int rest = T - nfull * 4 * NV;
    const int npass = nfull + (rest > 0);
    const int nv_last = rest <= 4 ? 1 : NV;
    const int split = nv_last == 1 && rest > 0 ? nfull : npass;   // passes before the one-tile pass
    // The last, partly filled pass (one tile per wave, or NV tiles for some waves) runs
    // first, after the first full pass or last, by workgroup (b % 3), so that the logits
    // stores at the ends of passes are not issued by every CU at the same moment.  lastp:
    // its logical index; sp: its position in the workgroup's stream of passes.
    const int lastp = rest > 0 ? nfull : npass;
    const int sp = lastp >= npass ? npass : (b % 3 == 1 ? 0 : (b % 3 == 2 ? min(1, lastp) : lastp));
    auto stream_pass = [&](int q) __attribute__((always_inline)) {   // logical pass of stream position q
        return lastp >= npass ? q : (q < sp ? q : (q == sp ? lastp : q - 1));
    };
    auto pass_first = [&](int p) __attribute__((always_inline)) {
        const int nv = p < nfull ? NV : nv_last;
        return t_begin + p * 4 * NV + wave * nv;
    };
    auto pass_count = [&](int p) __attribute__((always_inline)) {
        const int nv = p < nfull ? NV : nv_last;
        const int c = t_end - pass_first(p);
        return c < 0 ? 0 : (c < nv ? c : nv);
    };

    // ---- W: DMA instruction j of a step fills rows 8 j .. 8 j + 7 of the wave's part of a W slot
    const int lrow = lane >> 3;                  // row within an instruction's 1 KB block
    int wchunk[WJ];                               // logical chunk this lane fetches, per instruction
#pragma unroll
    for (int j = 0; j < WJ; ++j) wchunk[j] = (lane & 7) ^ swz(8 * j + lrow);
    u32x4 wbuf;
    int wvoff[WJ];
    int wp = 0, wks = 0;                         // W DMA cursor (pass, step); wp == npass: past the end
    auto set_w = [&](int p) __attribute__((always_inline)) {
        const int lp = stream_pass(p < npass ? p : npass - 1);
        const int cnt = p < npass ? pass_count(lp) : 0;
        const int base = min(pass_first(lp), a.tiles - 1) * 32;
        const int64_t rest_bytes = (int64_t)(a.V - base) * H * 2;
        const int64_t span = (int64_t)WR * H * 2;
        wbuf = sbuf(a.W + (int64_t)base * H, rest_bytes < span ? rest_bytes : span);
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            const int row = 8 * j + lrow;
            wvoff[j] = (row >> 5) < cnt ? row * H * 2 + wchunk[j] * 16 : kBig;
        }
    };
    auto issue_w = [&](uint32_t slot_lds) __attribute__((always_inline)) {
        const uint32_t dst = slot_lds + wave * (WR * 128);
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            if constexpr (HFULL) {
                dma16(wbuf, dst + j * 1024, wvoff[j], wks * (kBK * 2));
            } else {
                const bool ok = wks * 8 + wchunk[j] < hchunks;
                dma16(wbuf, dst + j * 1024, ok ? wvoff[j] + wks * (kBK * 2) : kBig, 0);
            }
        }
        if (++wks == nks) {
            wks = 0;
            ++wp;
            set_w(wp < npass ? wp : npass);
        }
    };

    // ---- hidden: instruction q of a wave fills rows (4 q + wave) * 8 .. + 7 of a hidden slot
    const int mrows = min(a.M - m0, HR);
    const u32x4 hbuf = sbuf(a.hidden + (int64_t)m0 * H, (int64_t)mrows * H * 2);
    int hvoff[MT], hchunk[MT];
#pragma unroll
    for (int q = 0; q < MT; ++q) {
        const int row = (4 * q + wave) * 8 + lrow;
        hchunk[q] = (lane & 7) ^ swz(row);
        hvoff[q] = row * H * 2 + hchunk[q] * 16;     // rows past the batch fall outside the range
    }
    int hks = 0;
    auto issue_h = [&](uint32_t slot_lds) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < MT; ++q) {
            const uint32_t dst = slot_lds + (4 * q + wave) * 1024;
            if constexpr (HFULL) {
                dma16(hbuf, dst, hvoff[q], hks * (kBK * 2));
            } else {
                const bool ok = hks * 8 + hchunk[q] < hchunks;
                dma16(hbuf, dst, ok ? hvoff[q] + hks * (kBK * 2) : kBig, 0);
            }
        }
        if (++hks == nks) hks = 0;
    };

    // fragment byte offsets within a slot: row 32 t + lr (t = tile), chunk (4 lh + s) ^ swz(row);
    // swz(32 t + lr) = swz(lr) ^ (4 (t & 1)), so two parities cover every tile
    int foff[2][4];
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int s = 0; s < 4; ++s) foff[par][s] = lr * 128 + (((4 * lh + s) ^ swz(lr) ^ (4 * par)) * 16);

    float run_m[MT], run_s[MT];     // running (max, sum exp) of the lane's half of its rows
#pragma unroll
    for (int i = 0; i < MT; ++i) { run_m[i] = -INFINITY; run_s[i] = 0.f; }
    // FILTER: a group of four logits is written only when its maximum reaches the row's
    // bound tau (at most the row's K-th largest logit, so no member of the top K is left out)
    float tau_r[FILTER ? MT : 1];
#pragma unroll
    for (int i = 0; i < (FILTER ? MT : 1); ++i) {
        const int m = m0 + i * 32 + lr;
        tau_r[i] = FILTER && m < a.M ? a.tau[m] : -INFINITY;
    }

    // ---- MFMAs of one step for NA tiles: W fragments first, then batch tiles, reads one tile ahead
    auto mfma_step = [&](auto& acc, uint32_t hs, uint32_t ws) __attribute__((always_inline)) {
        constexpr int NA = std::extent<std::remove_reference_t<decltype(acc)>>::value;
        const uint8_t* hsp = smem + (hs - lds0);
        const uint8_t* wsp = smem + (ws - lds0) + wave * (WR * 128);
        bf16x8 wf[NA][4];
#pragma unroll
        for (int v = 0; v < NA; ++v)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                wf[v][s] = *reinterpret_cast<const bf16x8*>(wsp + v * 4096 + foff[v & 1][s]);
        bf16x8 hb[2][4];
        auto read_frag = [&](int i, bf16x8 (&f)[4]) __attribute__((always_inline)) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                f[s] = *reinterpret_cast<const bf16x8*>(hsp + i * 4096 + foff[i & 1][s]);
        };
        read_frag(0, hb[0]);
        __builtin_amdgcn_sched_barrier(0);
        static_for<MT>([&](auto I) __attribute__((always_inline)) {
            constexpr int i = decltype(I)::value;
            if constexpr (i + 1 < MT) read_frag(i + 1, hb[(i + 1) & 1]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int v = 0; v < NA; ++v)
                    acc[v][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[v][s], hb[i & 1][s], acc[v][i], 0, 0, 0);
            if constexpr (i + 1 < MT) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4 * NA, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ---- pass epilogue: logits of the wave's tiles, the tile maxima and the running
    // (max, sum exp) of the batch rows.  Each lane keeps its own running pair for the 16
    // logits of a row it holds (online: the sum is rescaled when the maximum grows), and
    // the two lanes of a row are merged once at the end; a whole tile inside the
    // vocabulary takes a branch-free path.
    auto epilogue = [&](auto& acc, int p) __attribute__((always_inline)) {
        constexpr int NA = std::extent<std::remove_reference_t<decltype(acc)>>::value;
        constexpr float kL2E = 1.4426950408889634f;
        const int f = pass_first(p), cnt = pass_count(p);
#pragma unroll
        for (int v = 0; v < NA; ++v) {
            if (v < cnt) {
                const int tile = f + v;
                const int col = tile * 32 + 4 * lh;          // first logit of the lane, then +8 g + q
                const bool full = (tile + 1) * 32 <= a.V;
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const int m = m0 + i * 32 + lr;
                    // one accumulator at a time into VGPRs, where it is used
                    f32x16 z;
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        float x;
                        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(acc[v][i][j]));
                        z[j] = x;
                    }
                    if (!full) {
#pragma unroll
                        for (int j = 0; j < 16; ++j)
                            if (col + 8 * (j >> 2) + (j & 3) >= a.V) z[j] = -INFINITY;
                    }
                    uint32_t bits = 0;   // FILTER: groups 2 g + lh of the tile this lane wrote
                    if (m < a.M) {
                        float* dst = a.logits + (int64_t)m * a.ldz + col;
                        if (full) {
#pragma unroll
                            for (int g = 0; g < 4; ++g) {
                                bool put = true;
                                if constexpr (FILTER) {
                                    const float gm = fmaxf(fmaxf(z[4 * g], z[4 * g + 1]),
                                                           fmaxf(z[4 * g + 2], z[4 * g + 3]));
                                    put = gm >= tau_r[i];
                                    bits |= put ? 1u << (2 * g + lh) : 0u;
                                }
                                if (put)
                                    *reinterpret_cast<f32x4*>(dst + 8 * g) =
                                        f32x4{z[4 * g], z[4 * g + 1], z[4 * g + 2], z[4 * g + 3]};
                            }
                        } else {
                            bits = 0xFFu;   // the partly filled last tile is written whole
#pragma unroll
                            for (int j = 0; j < 16; ++j)
                                if (col + 8 * (j >> 2) + (j & 3) < a.V) dst[8 * (j >> 2) + (j & 3)] = z[j];
                        }
                    }
                    float mx = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])),
                                     fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
                    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(z[8], z[9]), fmaxf(z[10], z[11])),
                                         fmaxf(fmaxf(z[12], z[13]), fmaxf(z[14], z[15]))));
                    if (a.tmax) {
                        // lanes l and l ^ 32 hold the two halves of the row's tile
                        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                                          false, false);
                        const float tm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                        if (lh == 0 && m < a.M) a.tmax[(int64_t)m * a.ldt + tile] = tm;
                        if constexpr (FILTER) {
                            const auto sb = __builtin_amdgcn_permlane32_swap(bits, bits, false, false);
                            if (lh == 0 && m < a.M) a.tmask[(int64_t)m * a.ldt + tile] = (uint8_t)(sb[0] | sb[1]);
                        }
                    }
                    const float nm = fmaxf(run_m[i], mx);
                    if (full || nm != -INFINITY) {
                        const float nml = nm * kL2E;
                        float s0 = run_s[i] * __builtin_amdgcn_exp2f(run_m[i] * kL2E - nml), s1 = 0.f;
#pragma unroll
                        for (int j = 0; j < 16; j += 2) {
                            s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(z[j], kL2E, -nml));
                            s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(z[j + 1], kL2E, -nml));
                        }
                        run_s[i] = s0 + s1;
                        run_m[i] = nm;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int i = 0; i < MT; ++i) acc[v][i] = f32x16{};
        }
    };

    if (npass > 0) {
        const uint32_t hs_lds = lds0, ws_lds = lds0 + 2 * HSLOT;
        // prologue: W 0, hidden 0, W 1, so that at every step exactly the 8 W loads of
        // one later step were issued after the hidden chunk the step waits for
        set_w(0);
        for (int i = 0; i + 2 < SW; ++i) issue_w(ws_lds + i * WSLOT);
        issue_h(hs_lds);
        issue_w(ws_lds + (SW - 2) * WSLOT);
        int hsl = 0, wsl = 0;                    // slots of the current step (g % 2, g % SW)
        auto run = [&](auto NA_, int p0, int p1) __attribute__((always_inline)) {
            constexpr int NA = decltype(NA_)::value;
            f32x16 acc[NA][MT];
#pragma unroll
            for (int v = 0; v < NA; ++v)
#pragma unroll
                for (int i = 0; i < MT; ++i) acc[v][i] = f32x16{};
            for (int p = p0; p < p1; ++p) {
                for (int ks = 0; ks < nks; ++ks) {
                    // this wave's share of the hidden chunk of this step has landed (only the
                    // W loads of the step after next may still be in flight); after the barrier
                    // everyone's has, and the slots refilled below are no longer read
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(WJ));
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    const int wnext = wsl == 0 ? SW - 1 : wsl - 1;      // (g + SW - 1) % SW
                    issue_h(hs_lds + (hsl ^ 1) * HSLOT);
                    issue_w(ws_lds + wnext * WSLOT);
                    mfma_step(acc, hs_lds + hsl * HSLOT, ws_lds + wsl * WSLOT);
                    hsl ^= 1;
                    wsl = wsl == SW - 1 ? 0 : wsl + 1;
                }
                epilogue(acc, p);
            }
        };
        if (sp > 0) run(std::integral_constant<int, NV>{}, 0, sp);
        if (lastp < npass) {
            if (split < npass) run(std::integral_constant<int, 1>{}, lastp, npass);
            else run(std::integral_constant<int, NV>{}, lastp, npass);
        }
        if (sp < lastp) run(std::integral_constant<int, NV>{}, sp, lastp);
        // the loads issued past the last step write LDS: let them land before the workgroup ends
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        // merge the two halves of each row (an empty half has s = 0)
        float rm = run_m[i], rs = run_s[i];
        lse_merge(rm, rs, __shfl_xor(rm, 32), __shfl_xor(rs, 32));
        const int m = m0 + i * 32 + lr;
        if (lh == 0 && m < a.M)
            a.part[(int64_t)m * a.G * kRowsWaves + b * kRowsWaves + wave] = make_float2(rm, rs);
    }
}

template <int MT, int NV>
hipError_t launch_rows(const LmHeadArgs& a, dim3 grid, hipStream_t s) {
    if constexpr (NV > 1) {
        if (a.tau) {
            if (a.H % kBK == 0)
                hipLaunchKernelGGL((lmhead_dma_kernel<MT, true, NV, kWSlots, true>), grid, dim3(256), 0, s, a);
            else
                hipLaunchKernelGGL((lmhead_dma_kernel<MT, false, NV, kWSlots, true>), grid, dim3(256), 0, s, a);
            return hipGetLastError();
        }
    }
    if (a.H % kBK == 0)
        hipLaunchKernelGGL((lmhead_dma_kernel<MT, true, NV>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((lmhead_dma_kernel<MT, false, NV>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

// Row chunks of up to 256 rows (eight 32-row tiles: 256 AGPRs of accumulators
// and all 160 KB of LDS); up to 64 rows one vocab tile per wave and pass.
constexpr int kMaxChunkRows = 256;
int vocab_tiles_per_wave(int M) { return M <= 64 ? 1 : kNV; }
int row_chunks(int M) { return M <= kMaxChunkRows ? 1 : (M + kMaxChunkRows - 1) / kMaxChunkRows; }
int chunk_tiles(int M) {   // 32-row tiles per chunk
    const int gy = row_chunks(M);
    return ((M + gy - 1) / gy + 31) / 32;
}
// workgroups along the vocabulary: one per CU (256 on MI355X) over all row chunks
int lmhead_grid(int M, int V) {
    const int tiles = (V + 31) / 32;
    const int per_pass = 4 * vocab_tiles_per_wave(M);
    const int need = (tiles + per_pass - 1) / per_pass;
    const int cap = 256 / row_chunks(M) > 0 ? 256 / row_chunks(M) : 1;
    return need < cap ? need : cap;
}

// ---------------------------------------------------------------- the sample of the filter
// The exact logits of S vocabulary tiles (tile floor(j T / S) for j < S, T tiles; all
// full when T >= 4 S) for every row, by the same MFMA sequence as lmhead_dma_kernel: for
// each 64-wide step ks and sub-step s, lane l of the wave feeds W row l % 32 and batch
// row l % 32 with reduction indices 64 ks + 32 (l / 32) + 8 s .. + 7 (zero past H), into
// one accumulator per 32 x 32 tile, in that order.  So every sample logit equals the
// main kernel's logit of the same row and vocabulary id bit for bit, and the K-th
// largest sample logit of a row is at most the row's K-th largest logit.
// One wave per (sampled tile, 32-row batch tile); fragments come straight from memory.
constexpr int kSampleTiles = 128;
__global__ void __launch_bounds__(64) lmhead_sample_kernel(const uint16_t* __restrict__ hidden,
                                                           const uint16_t* __restrict__ W, int M, int H,
                                                           int tiles, int S, float* __restrict__ zs,
                                                           int64_t ldzs) {
    const int j = blockIdx.x, i = blockIdx.y;
    const int lane = threadIdx.x, lr = lane & 31, lh = lane >> 5;
    const int t = (int)((int64_t)j * tiles / S);
    const int mrow = i * 32 + lr;
    const bool hrow = mrow < M;
    const bf16x8* wp = reinterpret_cast<const bf16x8*>(W + ((int64_t)t * 32 + lr) * H);
    const bf16x8* hp = reinterpret_cast<const bf16x8*>(hidden + (int64_t)(hrow ? mrow : 0) * H);
    const int hchunks = H / 8, nks = (H + kBK - 1) / kBK;
    const bf16x8 zero = {};
    f32x16 acc = f32x16{};
    // a ring of kRing steps of fragments in registers: the loads of step ks + kRing are issued
    // as soon as step ks has been multiplied, so the one accumulator chain never waits for
    // more than the latency of a load spread over kRing steps
    constexpr int kRing = 8;
    bf16x8 wf[kRing][4], hf[kRing][4];
    auto load = [&](int ks, bf16x8 (&w)[4], bf16x8 (&h)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = 8 * ks + 4 * lh + s;       // 16-byte chunk of the row
            const bool ok = ks < nks && c < hchunks;
            w[s] = ok ? wp[c] : zero;
            h[s] = ok && hrow ? hp[c] : zero;
        }
    };
#pragma unroll
    for (int u = 0; u < kRing; ++u) load(u, wf[u], hf[u]);
    for (int k0 = 0; k0 < nks; k0 += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            if (k0 + u < nks) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[u][s], hf[u][s], acc, 0, 0, 0);
                load(k0 + u + kRing, wf[u], hf[u]);
            }
        }
    }
    // register r of lane l: vocabulary entry 8 (r / 4) + 4 (l / 32) + r % 4 of the tile, batch row l % 32
    if (hrow) {
        float* dst = zs + (int64_t)mrow * ldzs + j * 32 + 4 * lh;
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(dst + 8 * g) = f32x4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    }
}

// One (max, sum) partial per row and vocabulary workgroup (or wave) -> lse.
__global__ void __launch_bounds__(256) lse_combine_kernel(const float2* part, int nparts, float* lse, int M) {
    __shared__ float2 red[4];
    const float v = block_lse(part, blockIdx.x, nparts, red);
    if (threadIdx.x == 0) lse[blockIdx.x] = v;
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

int lmhead_partials(int M, int V) { return lmhead_grid(M, V) * kRowsWaves; }

int lmhead_sample_tiles(int M, int V) {
    const int tiles = (V + 31) / 32;
    return vocab_tiles_per_wave(M) > 1 && tiles >= 4 * kSampleTiles ? kSampleTiles : 0;
}

hipError_t launch_lmhead_sample(const uint16_t* hidden, const uint16_t* W, int M, int H, int V, int S, float* zs,
                                int64_t ldzs, hipStream_t s) {
    if (M <= 0 || S <= 0) return hipSuccess;
    hipLaunchKernelGGL(lmhead_sample_kernel, dim3(S, (M + 31) / 32), dim3(64), 0, s, hidden, W, M, H, (V + 31) / 32,
                       S, zs, ldzs);
    return hipGetLastError();
}

bool lmhead_has_tile_max(int M) { return M > 0; }

hipError_t launch_lmhead(const uint16_t* hidden, const uint16_t* W, float* logits, int64_t ldz,
                         float2* lse_part, float* tile_max, int64_t ldt, int M, int H, int V, hipStream_t s,
                         const float* tau, uint8_t* tile_mask) {
    if (M <= 0) return hipSuccess;
    LmHeadArgs a;
    a.hidden = hidden; a.W = W; a.logits = logits; a.part = lse_part; a.ldz = ldz;
    a.tmax = tile_max; a.ldt = ldt;
    // the filtered kernel needs tile maxima and masks, and runs only for more than 64 rows
    a.tau = tau && tile_max && tile_mask && vocab_tiles_per_wave(M) > 1 ? tau : nullptr;
    a.tmask = tile_mask;
    a.M = M; a.H = H; a.V = V;
    a.G = lmhead_grid(M, V);
    a.tiles = (V + 31) / 32;
    const dim3 grid(a.G, row_chunks(M));
    switch (chunk_tiles(M)) {
        case 1: return launch_rows<1, 1>(a, grid, s);
        case 2: return launch_rows<2, 1>(a, grid, s);
        case 3: return launch_rows<3, kNV>(a, grid, s);
        case 4: return launch_rows<4, kNV>(a, grid, s);
        case 5: return launch_rows<5, kNV>(a, grid, s);
        case 6: return launch_rows<6, kNV>(a, grid, s);
        case 7: return launch_rows<7, kNV>(a, grid, s);
        default: return launch_rows<8, kNV>(a, grid, s);
    }
}

hipError_t launch_lse_combine(const float2* lse_part, int nparts, float* lse, int M, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(lse_combine_kernel, dim3(M), dim3(256), 0, s, lse_part, nparts, lse, M);
    return hipGetLastError();
}

hipError_t launch_row_lse(const float* logits, int64_t ldz, float* lse, int M, int V, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(row_lse_kernel, dim3(M), dim3(256), 0, s, logits, ldz, lse, V);
    return hipGetLastError();
}

}  // namespace dflash
