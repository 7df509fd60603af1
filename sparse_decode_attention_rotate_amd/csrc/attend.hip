// Exact softmax attention over the selected tokens only.
//
// Loki (poster page, "TL;DR"; "Visual Insights", Figure 1 right): the
// full-dimensional keys of the k selected tokens give the final attention
// scores; softmax and the value sum run over those k tokens.
//   z_t = scale * sum_{j<D} qr_j krot_{t,j},  p = softmax(z) over idx,
//   out = sum_t p_t V_t.
//
// Split-k: workgroup (split, b*Hq+h) takes up to kAttendChunk selected rows,
// whose token indices it first stages in LDS.  A row is read by a group of LPR
// lanes, 16 bytes each (LPR = D*elem/16); each lane group walks its rows in
// batches of kRowsPerBatch, with the key and value loads of the next batch in
// flight while the current one is consumed (raw buffer loads: rows past the
// end or with invalid indices read as zeros, no branch).  Each lane group keeps
// an online softmax (running max m, sum l, weighted value acc); the groups are
// merged in LDS at the end.
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
constexpr int kRowsPerBatch = 4;  // rows per lane group per load batch

template <int DT, int D, bool SPLIT>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttendParams p) {
  constexpr int EB = Elem<DT>::kBytes;
  constexpr int E = Elem<DT>::kPerVec;
  constexpr int LPR = D * EB / 16;                 // lanes per row
  constexpr int RPI = 64 / LPR;                    // rows per wave instruction
  constexpr int NG = (kAttThreads / 64) * RPI;     // lane groups per workgroup
  constexpr int RB = kRowsPerBatch;
  constexpr int ROWS_PER_ITER = 2 * RB * NG;       // two batches in flight

  __shared__ int sidx[kAttendChunk];
  __shared__ float slow[kAttendChunk];
  __shared__ float red_m[NG], red_l[NG];
  __shared__ float accs[NG][D];

  const Shape& sh = p.sh;
  const int split = blockIdx.x % p.nsplit;
  const size_t bh = blockIdx.x / p.nsplit;
  const int b = (int)(bh / sh.Hq), h = (int)(bh % sh.Hq);
  const size_t head = (size_t)b * sh.Hkv + h / sh.g;
  const int r0 = split * p.kc;
  const int nr = min(p.kc, p.k - r0);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave * RPI + lane / LPR;
  const int c = lane % LPR;  // 16-byte chunk of a row: dims [c*E, c*E+E)
  const int j0 = c * E;

  // the chunk's token indices (invalid ones as -1) and low-dim partial logits
  for (int r = tid; r < nr; r += kAttThreads) {
    const int t = p.idx[bh * p.k + r0 + r];
    sidx[r] = (t >= 0 && t < sh.S) ? t : -1;
    if (SPLIT) slow[r] = p.sel_scores[bh * p.k + r0 + r] * p.scale_log2;
  }

  // qr slice, pre-multiplied by scale*log2(e); in the split variant the
  // coordinates below dp are already in the low-dim partial logit.
  float qv[E];
  const float* qrow = p.qr + bh * D;
#pragma unroll
  for (int e = 0; e < E; e++) {
    const int j = j0 + e;
    const float v = qrow[j] * p.scale_log2;
    qv[e] = (SPLIT && j < sh.dp) ? 0.f : v;
  }
  // byte offset of this lane's key chunk inside a row's part of the cache
  const bool k_needed = !SPLIT || j0 >= sh.dp;
  const bool in_panel = j0 < sh.dp;
  const uint32_t k_row_bytes = (uint32_t)((in_panel ? sh.dp : sh.kl.rest) * EB);
  const uint32_t k_base = (uint32_t)((in_panel ? (size_t)j0 : sh.kl.rest_off + (j0 - sh.dp)) * EB);
  const Rsrc krs = make_rsrc(static_cast<const char*>(p.kcache) + head * sh.kl.head_elems * EB,
                             (uint32_t)(sh.kl.head_elems * EB));
  const Rsrc vrs = make_rsrc(static_cast<const char*>(p.vcache) + head * (size_t)sh.S_cap * D * EB,
                             (uint32_t)((size_t)sh.S_cap * D * EB));
  __syncthreads();

  float m = -INFINITY, l = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; e++) acc[e] = 0.f;

  auto issue = [&](u32x4 (&kb)[RB], u32x4 (&vb)[RB], int rbase) {
#pragma unroll
    for (int q = 0; q < RB; q++) {
      const int r = rbase + q * NG;
      const int t = r < nr ? sidx[r] : -1;
      kb[q] = load16(krs, (t >= 0 && k_needed) ? k_base + (uint32_t)t * k_row_bytes : kOutOfRange);
      vb[q] = load16(vrs, t >= 0 ? ((uint32_t)t * D + j0) * EB : kOutOfRange);
    }
  };
  auto consume = [&](const u32x4 (&kb)[RB], const u32x4 (&vb)[RB], int rbase) {
    float z[RB];
    float mb = -INFINITY;
#pragma unroll
    for (int q = 0; q < RB; q++) {
      float f[E];
      unpack16<DT>(kb[q], f);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < E; e++) a = fmaf(qv[e], f[e], a);
      a = group_sum<LPR>(a);
      const int r = rbase + q * NG;
      const bool ok = r < nr && sidx[r] >= 0;
      if (SPLIT && ok) a += slow[r];
      z[q] = ok ? a : -INFINITY;
      mb = fmaxf(mb, z[q]);
    }
    const float mn = fmaxf(m, mb);
    if (mn == -INFINITY) return;  // nothing valid yet in this lane group
    const float sc = exp2f(m - mn);  // m = -inf -> 0
    l *= sc;
#pragma unroll
    for (int e = 0; e < E; e++) acc[e] *= sc;
#pragma unroll
    for (int q = 0; q < RB; q++) {
      const float w = exp2f(z[q] - mn);  // -inf -> 0
      l += w;
      float f[E];
      unpack16<DT>(vb[q], f);
#pragma unroll
      for (int e = 0; e < E; e++) acc[e] = fmaf(w, f[e], acc[e]);
    }
    m = mn;
  };

  u32x4 ka[RB], va[RB], kb2[RB], vb2[RB];
  issue(ka, va, grp);
  for (int base = 0; base < nr; base += ROWS_PER_ITER) {
    issue(kb2, vb2, base + RB * NG + grp);
    consume(ka, va, base + grp);
    if (base + ROWS_PER_ITER < nr) issue(ka, va, base + ROWS_PER_ITER + grp);
    consume(kb2, vb2, base + RB * NG + grp);
  }

  // merge the lane groups
  if (c == 0) {
    red_m[grp] = m;
    red_l[grp] = l;
  }
#pragma unroll
  for (int e = 0; e < E; e++) accs[grp][j0 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float M = -INFINITY;
#pragma unroll
    for (int gi = 0; gi < NG; gi++) M = fmaxf(M, red_m[gi]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int gi = 0; gi < NG; gi++) {
      const float w = red_m[gi] == -INFINITY ? 0.f : exp2f(red_m[gi] - M);
      L = fmaf(red_l[gi], w, L);
      A = fmaf(accs[gi][tid], w, A);
    }
    if (p.nsplit == 1) {
      p.out[bh * D + tid] = A / L;
    } else {
      float* part = p.part + (bh * p.nsplit + split) * (size_t)(D + 2);
      part[2 + tid] = A;
      if (tid == 0) {
        part[0] = M;
        part[1] = L;
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
    const float w = ps[0] == -INFINITY ? 0.f : exp2f(ps[0] - M);
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
