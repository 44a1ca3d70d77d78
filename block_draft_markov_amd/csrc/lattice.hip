// Parts 3 and 4 of the draft step: the candidate scorer (one workgroup per
// position and request) and the walk (one workgroup per request, every request
// in one launch).  The device functions they run, and the pages they follow,
// are in lattice_dev.hpp.

#include "common.hpp"
#include "internal.hpp"
#include "lattice_dev.hpp"

namespace dflash {

namespace {

__global__ void __launch_bounds__(kPairThreads) pair_scores_kernel(PairArgs A) {
    __shared__ PairSmem s;
    const int p = blockIdx.x, req = blockIdx.y;
    int a, n;
    row_range(A.row_offsets, req, A.L, A.M, a, n);
    if (p >= n) return;
    pair_position(A, req, a, p, s);
}

__global__ void __launch_bounds__(kLatThreads) walk_kernel(WalkArgs A) {
    __shared__ WalkSmem s;
    walk_request(A, blockIdx.x, s);
}

}  // namespace

hipError_t launch_pair_scores(const int64_t* cand_tok, const float* tables, const float* gate_w,
                              const uint16_t* hidden, const int64_t* last_tok, const int32_t* row_offsets,
                              int R, int L, int M, int H, int Vt, int K, int r, float* pair, hipStream_t s) {
    if (R <= 0 || M <= 0) return hipSuccess;
    const PairArgs A{cand_tok, tables, gate_w, hidden, last_tok, row_offsets, L, M, H, Vt, K, r, pair};
    hipLaunchKernelGGL(pair_scores_kernel, dim3(L, R), dim3(kPairThreads), 0, s, A);
    return hipGetLastError();
}

hipError_t launch_walk(const int64_t* cand_tok, const float* unary, const float* pair, const int32_t* row_offsets,
                       int R, int L, int M, int K, int walk, int64_t* tokens, float* scores, int32_t* slots,
                       hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const WalkArgs A{cand_tok, unary, pair, row_offsets, L, M, K, walk, nullptr, 1.f, tokens, scores, slots, nullptr};
    hipLaunchKernelGGL(walk_kernel, dim3(R), dim3(kLatThreads), 0, s, A);
    return hipGetLastError();
}

hipError_t launch_walk_sampled(const int64_t* cand_tok, const float* unary, const float* pair,
                               const int32_t* row_offsets, int R, int L, int M, int K, const double* uniforms,
                               float temperature, int64_t* tokens, float* scores, int32_t* slots, double* q,
                               hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const WalkArgs A{cand_tok, unary, pair, row_offsets, L, M, K, kWalkSampled, uniforms, temperature, tokens,
                     scores, slots, q};
    hipLaunchKernelGGL(walk_kernel, dim3(R), dim3(kLatThreads), 0, s, A);
    return hipGetLastError();
}

}  // namespace dflash
