// Block-wide exact attention over a list of selected tokens (device code
// shared by the split-k attention kernel and the fused decode kernel).
//
// Loki (poster page, "TL;DR"; "Visual Insights", Figure 1 right): the
// full-dimensional keys of the selected tokens give the final attention
// scores; softmax and the value sum run over those tokens only.
//   z_t = scale * sum_{j<D} qr_j krot_{t,j},  p = softmax(z),  out = sum_t p_t V_t.
//
// A row is read by a group of LPR lanes, 16 bytes each (LPR = D*elem/16).
// Each lane group walks its rows in batches of kRowsPerBatch with the key and
// value loads of the next batch in flight while the current one is consumed
// (raw buffer loads: rows past the end or with invalid indices read as zeros,
// no branch), keeping an online softmax (running max m, sum l, weighted value
// acc).  The lane groups are merged in LDS at the end.
//
// Split variant (the leading dp coordinates were already multiplied during
// scoring and their partial logits are given): only the remaining D-dp key
// coordinates are read, z_t = scale * (s_low_t + sum_{j>=dp} qr_j krot_{t,j}).
//
// Low-dimensional variant (LOW, PCAAttn): the logits use only the leading
// kdim rotated coordinates, z_t = scale * sum_{j<kdim} qr_j krot_{t,j}; key
// chunks wholly past kdim are not read.
#pragma once

#include "loki_internal.h"
#include "select_core.h"

namespace loki {

constexpr int kRowsPerBatch = 4;  // default rows per lane group per load batch

// Lane geometry of a row of D elements: a power-of-two number of 16-byte
// lanes.  D = 96 takes the lanes of 128 elements; the lanes past D read
// nothing and contribute zeros.
template <int D>
constexpr int kLaneDim = D == 96 ? 128 : D;

template <int DT, int D, int NT>
struct AttendGeom {
  static constexpr int EB = Elem<DT>::kBytes;
  static constexpr int E = Elem<DT>::kPerVec;
  static constexpr int DL = kLaneDim<D>;          // row elements covered by the lanes
  static constexpr int LPR = DL * EB / 16;        // lanes per row
  static constexpr int RPI = 64 / LPR;            // rows per wave instruction
  static constexpr int NG = (NT / 64) * RPI;      // lane groups per workgroup
};

template <int DT, int D, int NT>
struct AttendSmem {
  float red_m[AttendGeom<DT, D, NT>::NG], red_l[AttendGeom<DT, D, NT>::NG];
  float accs[AttendGeom<DT, D, NT>::NG][AttendGeom<DT, D, NT>::DL];
};

__device__ __forceinline__ float low_logit(float v) { return v; }
__device__ __forceinline__ float low_logit(unsigned key) { return key_score(key); }

// All NT threads call this together.  qrow: the query in the rotated basis
// (fp32, global or LDS); sidx[0..nr): token indices in LDS, -1 = skip;
// slow[0..nr): low-dim partial logits in LDS (split variant only, unscaled),
// as floats or as their order keys (select_keys);
// head: flattened (b, kv) of the caches.  On return thread tid < D holds the
// merged (M, L, A) with A the unnormalised output coordinate tid, in the log2
// domain: out[tid] = A / L.
// STREAM: the rows are read once (one query head per KV head): nontemporal
// loads; else (several query heads read the same rows) default-policy loads,
// which keep the rows in L2 for the other heads.
template <int DT, int D, int NT, bool SPLIT, int RB = kRowsPerBatch, bool LOW = false,
          bool STREAM = true, typename Low = float>
__device__ __forceinline__ void block_attend(const float* qrow, float scale_log2,
                                             const int* sidx, const Low* slow, int nr,
                                             const void* kcache, const void* vcache,
                                             size_t head, const Shape& sh,
                                             AttendSmem<DT, D, NT>& sm, float& M_out,
                                             float& L_out, float& A_out, int kdim = D) {
  using G = AttendGeom<DT, D, NT>;
  constexpr int EB = G::EB, E = G::E, LPR = G::LPR, RPI = G::RPI, NG = G::NG;
  constexpr int ROWS_PER_ITER = 2 * RB * NG;  // two batches in flight

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave * RPI + lane / LPR;
  const int c = lane % LPR;  // 16-byte chunk of a row: dims [c*E, c*E+E)
  const int j0 = c * E;

  // qr slice, pre-multiplied by scale*log2(e); in the split variant the
  // coordinates below dp are already in the low-dim partial logit.  Lanes
  // past the row (D = 96) hold zeros and read nothing.
  const bool in_row = j0 < D;
  float qv[E];
#pragma unroll
  for (int e = 0; e < E; e++) {
    const int j = j0 + e;
    const float v = in_row ? qrow[j] * scale_log2 : 0.f;
    qv[e] = ((SPLIT && j < sh.dp) || (LOW && j >= kdim)) ? 0.f : v;
  }
  // byte offset of this lane's key chunk inside a row's part of the cache
  const bool k_needed = in_row && (!SPLIT || j0 >= sh.dp) && (!LOW || j0 < kdim);
  const bool in_panel = j0 < sh.dp;
  const uint32_t k_row_bytes = (uint32_t)((in_panel ? sh.dp : sh.kl.rest) * EB);
  const uint32_t k_base = (uint32_t)((in_panel ? (size_t)j0 : sh.kl.rest_off + (j0 - sh.dp)) * EB);
  const Rsrc krs = make_rsrc(static_cast<const char*>(kcache) + head * sh.kl.head_elems * EB,
                             (uint32_t)(sh.kl.head_elems * EB));
  const Rsrc vrs = make_rsrc(static_cast<const char*>(vcache) + head * (size_t)sh.S_cap * D * EB,
                             (uint32_t)((size_t)sh.S_cap * D * EB));

  float m = -INFINITY, l = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; e++) acc[e] = 0.f;

  auto issue = [&](u32x4 (&kb)[RB], u32x4 (&vb)[RB], int rbase) {
#pragma unroll
    for (int q = 0; q < RB; q++) {
      const int r = rbase + q * NG;
      const int t = r < nr ? sidx[r] : -1;
      const uint32_t ko = (t >= 0 && k_needed) ? k_base + (uint32_t)t * k_row_bytes : kOutOfRange;
      const uint32_t vo = (t >= 0 && in_row) ? ((uint32_t)t * D + j0) * EB : kOutOfRange;
      kb[q] = STREAM ? load16_stream(krs, ko) : load16(krs, ko);
      vb[q] = STREAM ? load16_stream(vrs, vo) : load16(vrs, vo);
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
      if (SPLIT && ok) a = fmaf(low_logit(slow[r]), scale_log2, a);
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

  // Every batch is issued, also past the last row (those loads are out of
  // range: zeros, no memory access), so that the loads in flight are the same
  // on every path and each use waits only for its own batch; the scheduling
  // barriers keep each batch's use after the issue of the next one.
  u32x4 ka[RB], va[RB], kb2[RB], vb2[RB];
  issue(ka, va, grp);
  for (int base = 0; base < nr; base += ROWS_PER_ITER) {
    issue(kb2, vb2, base + RB * NG + grp);
    __builtin_amdgcn_sched_barrier(0);
    consume(ka, va, base + grp);
    issue(ka, va, base + ROWS_PER_ITER + grp);
    __builtin_amdgcn_sched_barrier(0);
    consume(kb2, vb2, base + RB * NG + grp);
  }

  // merge the lane groups
  if (c == 0) {
    sm.red_m[grp] = m;
    sm.red_l[grp] = l;
  }
#pragma unroll
  for (int e = 0; e < E; e++) sm.accs[grp][j0 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float M = -INFINITY;
#pragma unroll
    for (int gi = 0; gi < NG; gi++) M = fmaxf(M, sm.red_m[gi]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int gi = 0; gi < NG; gi++) {
      const float w = sm.red_m[gi] == -INFINITY ? 0.f : exp2f(sm.red_m[gi] - M);
      L = fmaf(sm.red_l[gi], w, L);
      A = fmaf(sm.accs[gi][tid], w, A);
    }
    M_out = M;
    L_out = L;
    A_out = A;
  }
}

// Merge of two partial results (M, L, A) of disjoint row sets of one query
// row (log2 domain, A unnormalised): the output coordinate.
__device__ __forceinline__ float combine_partials(float M0, float L0, float A0, float M1, float L1,
                                                  float A1) {
  const float M = fmaxf(M0, M1);
  const float w0 = M0 == -INFINITY ? 0.f : exp2f(M0 - M);
  const float w1 = M1 == -INFINITY ? 0.f : exp2f(M1 - M);
  return fmaf(A0, w0, A1 * w1) / fmaf(L0, w0, L1 * w1);
}

}  // namespace loki
