// Exact softmax attention over the selected tokens only.
//
// Loki (poster page, "TL;DR"; "Visual Insights", Figure 1 right): the
// full-dimensional keys of the k selected tokens give the final attention
// scores; softmax and the value sum run over those k tokens.
//   z_t = scale * sum_{j<D} qr_j krot_{t,j},  p = softmax(z) over idx,
//   out = sum_t p_t V_t.
//
// Split-k: workgroup (split, b*Hq+h) takes up to kAttendChunk selected rows.
// A row is read by a group of LPR lanes, 16 bytes each (LPR = D*elem/16), the
// key row and the value row issued together so both are in flight at once.
// Logits go to LDS; one wave takes their max and the exp2 sum; the value rows
// are weighted and summed per lane group, then across groups in LDS.
//
// Split variant (d == dp and the low-dim scores of the selected tokens are
// given): the leading dp coordinates were already multiplied during scoring,
// so only the remaining D-dp coordinates of each selected key are read and
// z_t = scale * (s_low_t + sum_{j>=dp} qr_j krot_{t,j}).
//
// With nsplit > 1 each workgroup writes (m, l, acc[D]) in the log2 domain and
// combine_kernel merges them.
#include "loki_internal.h"

namespace loki {

namespace {

constexpr int kAttThreads = 256;

template <int DT, int D, bool SPLIT>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttendParams p) {
  constexpr int EB = Elem<DT>::kBytes;
  constexpr int E = Elem<DT>::kPerVec;
  constexpr int LPR = D * EB / 16;       // lanes per row
  constexpr int RPI = 64 / LPR;          // rows per wave instruction
  constexpr int NG = (kAttThreads / 64) * RPI;  // lane groups per workgroup
  constexpr int RPG = kAttendChunk / NG;         // rows per lane group
  static_assert(kAttendChunk % NG == 0, "chunk must split evenly over lane groups");

  __shared__ float zs[kAttendChunk];
  __shared__ float accs[NG][D];
  __shared__ float ml[2];

  const Shape& sh = p.sh;
  const int split = blockIdx.x % p.nsplit;
  const size_t bh = blockIdx.x / p.nsplit;
  const int b = (int)(bh / sh.Hq), h = (int)(bh % sh.Hq);
  const size_t head = (size_t)b * sh.Hkv + h / sh.g;
  const int r0 = split * p.kc;
  const int nr = min(p.kc, p.k - r0);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave * RPI + lane / LPR;
  const int c = lane % LPR;  // 16-byte chunk of the row: dims [c*E, c*E+E)
  const int j0 = c * E;

  // qr slice, pre-multiplied by scale*log2(e); in the split variant the
  // coordinates below dp are already in s_low and are masked out.
  float qv[E];
  const float* qrow = p.qr + bh * D;
#pragma unroll
  for (int e = 0; e < E; e++) {
    const int j = j0 + e;
    qv[e] = (SPLIT && j < sh.dp) ? 0.f : qrow[j] * p.scale_log2;
  }
  const bool k_chunk_needed = !SPLIT || j0 >= sh.dp;

  const char* kbase = static_cast<const char*>(p.kcache) + head * sh.kl.head_elems * EB;
  const char* vbase = static_cast<const char*>(p.vcache) + head * (size_t)sh.S_cap * D * EB;
  const int32_t* irow = p.idx + bh * p.k + r0;

  // token of each row this lane group owns; -1 past the chunk end and for
  // indices outside [0, S) (those rows get zero weight)
  int tok[RPG];
  u32x4 kx[RPG], vx[RPG];
#pragma unroll
  for (int u = 0; u < RPG; u++) {
    const int r = grp + u * NG;
    int t = (r < nr) ? irow[r] : -1;
    tok[u] = (t >= 0 && t < sh.S) ? t : -1;
  }
#pragma unroll
  for (int u = 0; u < RPG; u++) {
    kx[u] = u32x4{0u, 0u, 0u, 0u};
    vx[u] = u32x4{0u, 0u, 0u, 0u};
    if (tok[u] >= 0) {
      const size_t t = (size_t)tok[u];
      if (k_chunk_needed) {
        const size_t off = (j0 < sh.dp) ? t * sh.dp + j0
                                        : sh.kl.rest_off + t * sh.kl.rest + (j0 - sh.dp);
        kx[u] = *reinterpret_cast<const u32x4*>(kbase + off * EB);
      }
      vx[u] = *reinterpret_cast<const u32x4*>(vbase + (t * D + j0) * EB);
    }
  }

  const float* slow = SPLIT ? p.sel_scores + bh * p.k + r0 : nullptr;
#pragma unroll
  for (int u = 0; u < RPG; u++) {
    float f[E];
    unpack16<DT>(kx[u], f);
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < E; e++) a = fmaf(qv[e], f[e], a);
    a = group_sum<LPR>(a);
    const int r = grp + u * NG;
    if (c == 0 && r < nr) {
      if (SPLIT && tok[u] >= 0) a = fmaf(slow[r], p.scale_log2, a);
      zs[r] = tok[u] >= 0 ? a : -INFINITY;
    }
  }
  __syncthreads();

  if (wave == 0) {
    float m = -INFINITY;
    for (int r = lane; r < nr; r += 64) m = fmaxf(m, zs[r]);
    m = wave_max(m);
    float l = 0.f;
    for (int r = lane; r < nr; r += 64) l += exp2f(zs[r] - m);
    l = wave_sum(l);
    if (lane == 0) {
      ml[0] = m;
      ml[1] = l;
    }
  }
  __syncthreads();
  const float m = ml[0];

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; e++) acc[e] = 0.f;
#pragma unroll
  for (int u = 0; u < RPG; u++) {
    if (tok[u] >= 0) {
      const float w = exp2f(zs[grp + u * NG] - m);
      float f[E];
      unpack16<DT>(vx[u], f);
#pragma unroll
      for (int e = 0; e < E; e++) acc[e] = fmaf(w, f[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; e++) accs[grp][j0 + e] = acc[e];
  __syncthreads();

  if (tid < D) {
    float s = 0.f;
#pragma unroll 8
    for (int gi = 0; gi < NG; gi++) s += accs[gi][tid];
    if (p.nsplit == 1) {
      p.out[bh * D + tid] = s / ml[1];
    } else {
      float* part = p.part + (bh * p.nsplit + split) * (size_t)(D + 2);
      part[2 + tid] = s;
      if (tid == 0) {
        part[0] = m;
        part[1] = ml[1];
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void combine_kernel(AttendParams p) {
  const size_t bh = blockIdx.x;
  const float* part = p.part + bh * p.nsplit * (size_t)(D + 2);
  float M = -INFINITY;
  for (int s = 0; s < p.nsplit; s++) M = fmaxf(M, part[s * (D + 2)]);
  float L = 0.f, a = 0.f;
  for (int s = 0; s < p.nsplit; s++) {
    const float* ps = part + s * (D + 2);
    const float w = exp2f(ps[0] - M);
    L = fmaf(ps[1], w, L);
    a = fmaf(ps[2 + threadIdx.x], w, a);
  }
  p.out[bh * D + threadIdx.x] = a / L;
}

template <int DT, int D>
hipError_t launch_d(const AttendParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.nsplit * p.sh.B * p.sh.Hq));
  if (p.sel_scores)
    attend_kernel<DT, D, true><<<grid, kAttThreads, 0, st>>>(p);
  else
    attend_kernel<DT, D, false><<<grid, kAttThreads, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  combine_kernel<D><<<dim3((unsigned)(p.sh.B * p.sh.Hq)), D, 0, st>>>(p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const AttendParams& p, hipStream_t st) {
  return p.sh.D == 128 ? launch_d<DT, 128>(p, st) : launch_d<DT, 64>(p, st);
}

}  // namespace

hipError_t launch_attend(const AttendParams& p, hipStream_t st) {
  switch (p.sh.dtype) {
    case F32: return launch_dt<F32>(p, st);
    case F16: return launch_dt<F16>(p, st);
    default: return launch_dt<BF16>(p, st);
  }
}

}  // namespace loki
