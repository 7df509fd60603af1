// Query rotation and key append: row vectors times the PCA basis P.
//
// Loki (NeurIPS 2024 poster page, "Visual Insights", Figure 1 right): keys are
// kept in the PCA basis found offline, and the query is brought into the same
// basis at inference so that its leading coordinates can score the cached
// keys.  The same product projects a newly appended key before it is written
// into the rotated cache (poster page, "Loki's Computational Cost": the
// KV-cache append is part of every decode step).
//
// One workgroup per (KV head, block of batch rows): P[kv] (fp32) is staged in
// LDS with 16-byte loads all in flight at once, the g query rows of each batch
// entry (and the new key, when appending) are staged as fp32, and each thread
// forms one output coordinate for its rows.
#include "loki_internal.h"

namespace loki {

namespace {

constexpr int kProjThreads = 256;
constexpr int kMaxRows = 32;

template <int DT, int D, int ACC>
__global__ __launch_bounds__(kProjThreads) void project_kernel(ProjectParams p) {
  constexpr int RG = kProjThreads / D;             // row groups
  constexpr int PV = D * D / 4 / kProjThreads;     // 16-byte pieces of P per thread
  static_assert(ACC * RG <= kMaxRows, "row buffer too small");
  __shared__ float xs[kMaxRows][D];
  __shared__ float ps[D * D];

  const Shape& sh = p.sh;
  const int kv = blockIdx.x;
  const int b0 = blockIdx.y * p.bb;
  const int nb = min(p.bb, sh.B - b0);
  const int nq = p.q ? sh.g : 0;
  const int per_b = nq + (p.k_new ? 1 : 0);
  const int R = nb * per_b;

  // P[kv] -> LDS: every 16-byte load issued before the first is consumed
  const u32x4* Pk = reinterpret_cast<const u32x4*>(p.P + (size_t)kv * D * D);
  u32x4 pv[PV];
#pragma unroll
  for (int u = 0; u < PV; u++) pv[u] = Pk[u * kProjThreads + threadIdx.x];

  // rows (queries, then the new key) as fp32; rows >= R are zero
  for (int e = threadIdx.x; e < ACC * RG * D; e += kProjThreads) {
    const int r = e / D, i = e % D;
    float x = 0.f;
    if (r < R) {
      const int b = b0 + r / per_b, which = r % per_b;
      if (which < nq)
        x = load_elem<DT>(p.q, ((size_t)b * sh.Hq + (size_t)kv * sh.g + which) * D + i);
      else
        x = load_elem<DT>(p.k_new, ((size_t)b * sh.Hkv + kv) * D + i);
    }
    xs[r][i] = x;
  }
#pragma unroll
  for (int u = 0; u < PV; u++)
    reinterpret_cast<u32x4*>(ps)[u * kProjThreads + threadIdx.x] = pv[u];
  __syncthreads();

  // thread (j, rg) forms coordinate j of rows rg, rg + RG, ...: branch-free
  // (D = 96: the threads past RG*D have no coordinate)
  static_assert(D * D % (4 * kProjThreads) == 0, "P in whole 16-byte pieces per thread");
  const int j = threadIdx.x % D, rg = threadIdx.x / D;
  if (rg >= RG) return;  // no barrier follows
  float acc[ACC];
#pragma unroll
  for (int a = 0; a < ACC; a++) acc[a] = 0.f;
#pragma unroll 2
  for (int i = 0; i < D; i += 4) {
    const float p0 = ps[(i + 0) * D + j], p1 = ps[(i + 1) * D + j];
    const float p2 = ps[(i + 2) * D + j], p3 = ps[(i + 3) * D + j];
#pragma unroll
    for (int a = 0; a < ACC; a++) {
      const float4 x4 = *reinterpret_cast<const float4*>(&xs[rg + a * RG][i]);
      acc[a] = fmaf(x4.x, p0, acc[a]);
      acc[a] = fmaf(x4.y, p1, acc[a]);
      acc[a] = fmaf(x4.z, p2, acc[a]);
      acc[a] = fmaf(x4.w, p3, acc[a]);
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
    for (int e = threadIdx.x; e < nb * D; e += RG * D) {
      const int b = b0 + e / D, i = e % D;
      const size_t head = (size_t)b * sh.Hkv + kv;
      copy_elem<DT>(p.vcache, (head * sh.S_cap + (size_t)p.pos) * D + i, p.v_new, head * D + i);
    }
  }
}

template <int DT, int D>
hipError_t launch_d(const ProjectParams& p, dim3 grid, int rows) {
  constexpr int RG = kProjThreads / D;
  const int acc = (rows + RG - 1) / RG;
  hipStream_t st = p.stream;
  if (acc <= 1)
    project_kernel<DT, D, 1><<<grid, kProjThreads, 0, st>>>(p);
  else if (acc <= 2)
    project_kernel<DT, D, 2><<<grid, kProjThreads, 0, st>>>(p);
  else if (acc <= 4)
    project_kernel<DT, D, 4><<<grid, kProjThreads, 0, st>>>(p);
  else if (acc <= 8)
    project_kernel<DT, D, 8><<<grid, kProjThreads, 0, st>>>(p);
  else
    project_kernel<DT, D, kMaxRows / RG><<<grid, kProjThreads, 0, st>>>(p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const ProjectParams& p, dim3 grid, int rows) {
  switch (p.sh.D) {
    case 128: return launch_d<DT, 128>(p, grid, rows);
    case 96: return launch_d<DT, 96>(p, grid, rows);
    default: return launch_d<DT, 64>(p, grid, rows);
  }
}

}  // namespace

hipError_t launch_project(const ProjectParams& p0, hipStream_t st) {
  ProjectParams p = p0;
  const int per_b = (p.q ? p.sh.g : 0) + (p.k_new ? 1 : 0);
  if (per_b == 0) return hipSuccess;
  // one batch row per workgroup: P is re-read from L2 by each workgroup, and
  // more workgroups shorten the latency of this small step
  p.bb = 1;
  if (per_b > kMaxRows) return hipErrorInvalidValue;  // g too large for one workgroup
  dim3 grid(p.sh.Hkv, (p.sh.B + p.bb - 1) / p.bb);
  p.stream = st;
  const int rows = p.bb * per_b;
  switch (p.sh.dtype) {
    case F32: return launch_dt<F32>(p, grid, rows);
    case F16: return launch_dt<F16>(p, grid, rows);
    default: return launch_dt<BF16>(p, grid, rows);
  }
}

}  // namespace loki
