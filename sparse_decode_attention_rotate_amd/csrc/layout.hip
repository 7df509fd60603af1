// Conversion between row-major rotated keys [B, Hkv, n, D] and the split-panel
// key cache (leading dp coordinates of every token first, then the rest).
// Pure data movement; one thread per element.
#include "loki_internal.h"

namespace loki {

namespace {

template <int DT>
__global__ __launch_bounds__(256) void layout_kernel(LayoutParams p) {
  const Shape& sh = p.sh;
  const size_t total = (size_t)sh.B * sh.Hkv * p.n_tokens * sh.D;
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int j = (int)(e % sh.D);
  const size_t t = (e / sh.D) % (size_t)p.n_tokens;
  const size_t head = e / ((size_t)sh.D * p.n_tokens);
  const size_t ci = sh.kl.at(head, t, j);
  if (p.to_cache)
    copy_elem<DT>(p.dst, ci, p.src, e);
  else
    copy_elem<DT>(p.dst, e, p.src, ci);
}

}  // namespace

hipError_t launch_layout(const LayoutParams& p, hipStream_t st) {
  const size_t total = (size_t)p.sh.B * p.sh.Hkv * p.n_tokens * p.sh.D;
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + 255) / 256));
  switch (p.sh.dtype) {
    case F32: layout_kernel<F32><<<grid, 256, 0, st>>>(p); break;
    case F16: layout_kernel<F16><<<grid, 256, 0, st>>>(p); break;
    default: layout_kernel<BF16><<<grid, 256, 0, st>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace loki
