// Per-query top-k selection, written as a bitmask over the whole cache: one
// workgroup per query row (the selection routine is in topk_row.hpp).
//
// Each query keeps its top_k best-scored earlier tokens [aiaulis paras 2-3;
// devotd section 1 table, 2048 tokens] and the selection is applied as a
// mask over the whole cache rather than by gathering rows [aiaulis para 4;
// devotd section 2].
#include "topk_row.hpp"

namespace dsa {
namespace {

template <int NW, int EPT_R, int EPT_L>
__global__ __launch_bounds__(NW * 64) void topk_mask_kernel(TopkParams a) {
  __shared__ TopkShared<NW, EPT_L> sh;
  topk_select_row<NW, EPT_R, EPT_L>(a, blockIdx.x, blockIdx.y, sh);
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t st) {
  const int nmax = p.q_pos0 + p.T;  // longest candidate row in the call
  dim3 grid(p.T, p.B);
  // Rows are latency-bound chains of barriers and LDS histograms, so the
  // smallest workgroup that holds a row (keys in registers) wins: more rows
  // are then in flight per CU.
  if (nmax <= 2048)
    hipLaunchKernelGGL((topk_mask_kernel<4, 8, 0>), grid, dim3(256), 0, st, p);
  else if (nmax <= 4096)
    hipLaunchKernelGGL((topk_mask_kernel<4, 16, 0>), grid, dim3(256), 0, st, p);
  else if (nmax <= 8192)
    hipLaunchKernelGGL((topk_mask_kernel<4, 32, 0>), grid, dim3(256), 0, st, p);
  else if (nmax <= 16384)
    hipLaunchKernelGGL((topk_mask_kernel<8, 32, 0>), grid, dim3(512), 0, st, p);
  else if (nmax <= 32768)
    hipLaunchKernelGGL((topk_mask_kernel<16, 32, 0>), grid, dim3(1024), 0, st, p);
  else if (nmax <= kTopkMaxRow)
    hipLaunchKernelGGL((topk_mask_kernel<16, 32, 32>), grid, dim3(1024), 0, st, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dsa
