// Per-(batch, query head) top-k selection by approximate score.
//
// Loki (briefgpt.xyz abstract; poster page "TL;DR" and Figure 1 right): the
// tokens of the KV-cache are ranked by their low-dimensional scores and only
// the top k are kept for the exact attention.
//
// One workgroup per row of scores in global memory; the selection itself
// (linear-bin histogram, exact threshold, ordered compaction) is block_select
// in select_core.h.
#include "loki_internal.h"
#include "select_core.h"

namespace loki {

namespace {

template <int NT, int KREG>
__global__ __launch_bounds__(NT) void topk_kernel(TopkParams p) {
  __shared__ SelectSmem<NT / 64> sm;
  const int S = p.S, k = p.k;
  const float* srow = p.scores + (size_t)blockIdx.x * S;
  const Rsrc srs = make_rsrc(srow, (uint32_t)S * 4u);
  auto load_score = [&](int i) -> float {
    return __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(srs, i < S ? i * 4 : (int)kOutOfRange, 0, 0));
  };
  block_select<NT, KREG>(load_score, S, k, p.idx + (size_t)blockIdx.x * k,
                         p.sel_scores ? p.sel_scores + (size_t)blockIdx.x * k : nullptr, sm);
}

}  // namespace
hipError_t launch_topk(const TopkParams& p, int n_rows, hipStream_t st) {
  const dim3 grid((unsigned)n_rows);
  if (p.S <= 512 * 8)
    topk_kernel<512, 8><<<grid, 512, 0, st>>>(p);
  else if (p.S <= 1024 * 16)
    topk_kernel<1024, 16><<<grid, 1024, 0, st>>>(p);
  else if (p.S <= 1024 * 32)
    topk_kernel<1024, 32><<<grid, 1024, 0, st>>>(p);
  else
    topk_kernel<1024, 0><<<grid, 1024, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace loki
