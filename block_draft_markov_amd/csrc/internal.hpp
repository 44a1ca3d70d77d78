// Internal launch interface between the C ABI (abi.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dflash {

// ---------------------------------------------------------------- part 1: lm_head GEMM
// A workgroup owns a contiguous range of vocabulary tiles and keeps one
// (max, sum exp) partial per row and wave.
int lmhead_partials(int M, int V);       // (max, sum exp) partials per row
// The kernel can also store the maximum of every tile of 32 logits of every
// row: tile_max [M][ldt], ldt >= ceil(V / 32).
bool lmhead_has_tile_max(int M);
// With tau (a per-row lower bound of the K-th largest logit) and tile_mask, a kernel of
// more than 64 rows writes only the groups of four logits whose maximum reaches tau and
// records them in tile_mask [M][ldt] (bit q of a tile's byte: logits 4 q .. 4 q + 3 of the
// tile written); the partly filled last tile is written whole.
hipError_t launch_lmhead(const uint16_t* hidden, const uint16_t* W, float* logits, int64_t ldz,
                         float2* lse_part, float* tile_max, int64_t ldt, int M, int H, int V, hipStream_t s,
                         const float* tau = nullptr, uint8_t* tile_mask = nullptr);
// Vocabulary tiles sampled for tau (0: no filtered kernel for this shape: at most 64 rows, or
// fewer than 512 tiles), and the sample:
// zs [M][ldzs], ldzs >= 32 S, the exact logits of the sampled tiles.
int lmhead_sample_tiles(int M, int V);
hipError_t launch_lmhead_sample(const uint16_t* hidden, const uint16_t* W, int M, int H, int V, int S, float* zs,
                                int64_t ldzs, hipStream_t s);
// tau[m] = the K-th largest of the n sample logits of row m (n <= 4096).
hipError_t launch_sample_tau(const float* zs, int64_t ldzs, int n, int M, int K, float* tau, hipStream_t s);
// lse[m] from the partials of row m.
hipError_t launch_lse_combine(const float2* lse_part, int nparts, float* lse, int M, hipStream_t s);
// lse[m] straight from logits.
hipError_t launch_row_lse(const float* logits, int64_t ldz, float* lse, int M, int V, hipStream_t s);

// ---------------------------------------------------------------- part 2: Top-K
// Chunks of 16384 logits per row on the exact path of the Top-K (rows with heavy
// ties); that path merges nchunks * K entries in LDS.
int topk_tiles_chunks(int V);
// Top-K from the maxima of the 32-logit tiles (one workgroup per row; rows with
// heavy ties take an exact path over all their logits in the same launch).  The lse
// of a row is lse[m] when lse is given, else merged from its (max, sum exp) partials.
// With tile_mask and tau (from the filtered lm_head kernel) only the written groups of
// logits are read, and tau raises the row's threshold.
hipError_t launch_topk_tiles(const float* logits, int64_t ldz, const float* tile_max, int64_t ldt,
                             const float* lse, const float2* lse_part, int nparts, const int64_t* d2t, int M,
                             int V, int K, int32_t* cand_idx, int64_t* cand_tok, float* unary, hipStream_t s,
                             const uint8_t* tile_mask = nullptr, const float* tau = nullptr);
// tile_max [M][ldt]: the maximum of every 32-logit tile of every row of logits [M][ldz].
hipError_t launch_tile_max(const float* logits, int64_t ldz, int M, int V, float* tile_max, int64_t ldt,
                           hipStream_t s);

// Head-less drafting: per row the lowest draft id maximizing the scaled, soft-capped
// logit, from the tile maxima when given (ldt > 0), else from a scan of the row.
hipError_t launch_argmax(const float* logits, int64_t ldz, const float* tile_max, int64_t ldt,
                         const int64_t* d2t, int M, int V, float scale, float cap, int64_t* tokens,
                         float* values, hipStream_t s);

// ---------------------------------------------------------------- parts 3 and 4: lattice
hipError_t launch_pair_scores(const int64_t* cand_tok, const float* tables, const float* gate_w,
                              const uint16_t* hidden, const int64_t* last_tok,
                              const int32_t* row_offsets, int R, int L, int M, int H, int Vt,
                              int K, int r, float* pair, hipStream_t s);
// The dense Markov walk: per position every request's scaled, soft-capped row biased by
// <A[previous token], B[t(v)]> and its lowest-id argmax; best [L][R] packed entries.
hipError_t launch_dense_walk(const float* logits, int64_t ldz, const int64_t* d2t, const float* tables,
                             const int64_t* last_tok, const int32_t* row_offsets, int R, int L, int M, int V,
                             int Vt, int r, float scale, float cap, uint64_t* best, int64_t* tokens, float* values,
                             hipStream_t s);
hipError_t launch_walk(const int64_t* cand_tok, const float* unary, const float* pair,
                       const int32_t* row_offsets, int R, int L, int M, int K, int walk,
                       int64_t* tokens, float* scores, int32_t* slots, hipStream_t s);
// The sampled walk: one double uniform per row, temperature > 0; q [M][K] (or NULL)
// receives the proposal of every row.
hipError_t launch_walk_sampled(const int64_t* cand_tok, const float* unary, const float* pair,
                               const int32_t* row_offsets, int R, int L, int M, int K, const double* uniforms,
                               float temperature, int64_t* tokens, float* scores, int32_t* slots, double* q,
                               hipStream_t s);

}  // namespace dflash
