// Query rotation and key append: row vectors times the PCA basis P.
//
// Loki (NeurIPS 2024 poster page, "Visual Insights", Figure 1 right): keys are
// kept in the PCA basis found offline, and the query is brought into the same
// basis at inference so that its leading coordinates can score the cached
// keys.  The same product projects a newly appended key before it is written
// into the rotated cache (poster page, "Loki's Computational Cost": the
// KV-cache append is part of every decode step).
//
// One workgroup per (KV head, block of batch rows): the g query rows of each
// batch entry (and the new key, when appending) are staged in LDS as fp32 and
// multiplied by P[kv], read once per workgroup with coalesced 512-byte rows.
#include "loki_internal.h"

namespace loki {

namespace {

constexpr int kProjThreads = 256;
constexpr int kMaxRows = 32;

template <int DT, int D>
__global__ __launch_bounds__(kProjThreads) void project_kernel(ProjectParams p) {
  constexpr int RG = kProjThreads / D;  // row groups
  constexpr int ACC = kMaxRows / RG;
  __shared__ float xs[kMaxRows][D];

  const Shape& sh = p.sh;
  const int kv = blockIdx.x;
  const int b0 = blockIdx.y * p.bb;
  const int nb = min(p.bb, sh.B - b0);
  const int nq = p.q ? sh.g : 0;
  const int per_b = nq + (p.k_new ? 1 : 0);
  const int R = nb * per_b;

  for (int e = threadIdx.x; e < R * D; e += kProjThreads) {
    const int r = e / D, i = e % D;
    const int b = b0 + r / per_b, which = r % per_b;
    float x;
    if (which < nq)
      x = load_elem<DT>(p.q, ((size_t)b * sh.Hq + (size_t)kv * sh.g + which) * D + i);
    else
      x = load_elem<DT>(p.k_new, ((size_t)b * sh.Hkv + kv) * D + i);
    xs[r][i] = x;
  }
  __syncthreads();

  const int j = threadIdx.x % D, rg = threadIdx.x / D;
  float acc[ACC];
#pragma unroll
  for (int a = 0; a < ACC; a++) acc[a] = 0.f;
  const float* Pk = p.P + (size_t)kv * D * D;
  for (int i = 0; i < D; i++) {
    const float pij = Pk[(size_t)i * D + j];
#pragma unroll
    for (int a = 0; a < ACC; a++) {
      const int r = rg + a * RG;
      if (r < R) acc[a] = fmaf(xs[r][i], pij, acc[a]);
    }
  }

#pragma unroll
  for (int a = 0; a < ACC; a++) {
    const int r = rg + a * RG;
    if (r < R) {
      const int b = b0 + r / per_b, which = r % per_b;
      if (which < nq) {
        p.qr[((size_t)b * sh.Hq + (size_t)kv * sh.g + which) * D + j] = acc[a];
      } else {
        const size_t head = (size_t)b * sh.Hkv + kv;
        store_elem<DT>(p.kcache, sh.kl.at(head, (size_t)p.pos, j), acc[a]);
      }
    }
  }

  if (p.k_new) {
    for (int e = threadIdx.x; e < nb * D; e += kProjThreads) {
      const int b = b0 + e / D, i = e % D;
      const size_t head = (size_t)b * sh.Hkv + kv;
      copy_elem<DT>(p.vcache, (head * sh.S_cap + (size_t)p.pos) * D + i, p.v_new, head * D + i);
    }
  }
}

template <int DT>
hipError_t launch_dt(const ProjectParams& p, dim3 grid, hipStream_t st) {
  if (p.sh.D == 128)
    project_kernel<DT, 128><<<grid, kProjThreads, 0, st>>>(p);
  else
    project_kernel<DT, 64><<<grid, kProjThreads, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_project(const ProjectParams& p0, hipStream_t st) {
  ProjectParams p = p0;
  const int per_b = (p.q ? p.sh.g : 0) + (p.k_new ? 1 : 0);
  if (per_b == 0) return hipSuccess;
  // a few batch rows per workgroup: P is re-read from L2 by each workgroup,
  // and more workgroups shorten the latency of this small step
  p.bb = kMaxRows / per_b;
  if (p.bb > 4) p.bb = 4;
  if (p.bb > p.sh.B) p.bb = p.sh.B;
  if (p.bb < 1) return hipErrorInvalidValue;  // g too large for one workgroup
  dim3 grid(p.sh.Hkv, (p.sh.B + p.bb - 1) / p.bb);
  switch (p.sh.dtype) {
    case F32: return launch_dt<F32>(p, grid, st);
    case F16: return launch_dt<F16>(p, grid, st);
    default: return launch_dt<BF16>(p, grid, st);
  }
}

}  // namespace loki
