// Internal declarations of the pair-statistics reduction (host planner and
// kernels): sum a*b, sum a*a, sum b*b of equal-shaped matrix pairs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace himuon {

// ---- pair statistics (sum a b, sum a a, sum b b of two equal-shaped matrices)
constexpr int kPairGroup = 256;   // matrix pairs per launch (kernel-argument table, ~14 KB)
struct PairEntry {
    const void* a;
    const void* b;
    int64_t lda, ldb;
    int32_t rows, cols;
    int32_t rows_per_block;   // rows one workgroup reduces
    int32_t nblocks;          // workgroups of this pair
    int32_t block_base;       // first workgroup of this pair in the launch
    int32_t part_base;        // first partial (3 doubles each) of this pair in the workspace
};
struct PairArgs {
    PairEntry e[kPairGroup];
    int32_t n;                // pairs in this launch
    int32_t total_blocks;     // workgroups of the partial-sum launch
    int32_t dtype;            // 0 bf16, 1 fp32
    double* partial;          // workspace: 3 doubles per workgroup
    double* out;              // 3 doubles per pair of this launch
};
hipError_t launch_pair_stats(const PairArgs& a, hipStream_t s);

}  // namespace himuon
