// Block-wide exact top-k selection (device code shared by the stand-alone
// top-k kernel and the fused decode kernel).
//
// Loki (briefgpt.xyz abstract; poster page "TL;DR" and Figure 1 right): the
// tokens of the KV-cache are ranked by their low-dimensional scores and only
// the top k are kept for the exact attention.
//
// Exact selection in one workgroup per row of S scores, rule (score
// descending, index ascending), output in ascending index order:
//  1. Linear binning.  bin(s) = floor((s - min) * 2047 / (max - min)) is a
//     non-decreasing function of s, so every score in a higher bin exceeds
//     every score in a lower one.  One LDS histogram of 2048 bins (spread
//     data, few atomic collisions) and a DPP prefix scan over the bins in
//     descending order give the bin b* that holds the k-th largest score.
//  2. Exact threshold inside b*.  With few members (<= 64) one wave ranks
//     them by (key, index) and reads off the threshold key T and the number r
//     of keys equal to T that are taken.  Otherwise (skewed rows) radix passes
//     over 8-bit digits of the members' order-preserving keys, per-wave LDS
//     histograms, early stop once a digit group is taken whole.
//  3. Ordered compaction: select key > T, or key == T among the first r such
//     indices.  Each wave owns a contiguous index range: counts by ballot, one
//     barrier to exchange them, then each wave writes its indices at offsets
//     from ballot + mbcnt ranks.
// Scores stay in registers when S <= threads * KREG, else they are re-read
// (from L2: the row was just written) in each step.
#pragma once

#include <limits.h>

#include "loki_common.h"

namespace loki {

constexpr int kBins = 2048;
constexpr int kFewCandidates = 64;

__device__ __forceinline__ unsigned order_key(float s) {
  unsigned u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lin_bin(float s, float lo, float scale) {
  const int b = (int)((s - lo) * scale);
  return b < 0 ? 0 : (b > kBins - 1 ? kBins - 1 : b);
}

// LDS scratch of one block_select call.
template <int NW>
struct SelectSmem {
  unsigned hist[kBins];
  unsigned whist[NW][256];
  float wmin[NW], wmax[NW];
  unsigned wtot[NW];
  int sel_bin, sel_gt, sel_eq, n_cand;
  unsigned cand_key[kFewCandidates];
  int cand_idx[kFewCandidates];
  unsigned thr_key, r_digit, r_gt, r_eq;
  int thr_take;
  int wcnt[NW][2];
};

// All NT threads of the workgroup call this together.  load_score(i) returns
// score i for 0 <= i < S and is harmless (any value) for i >= S.  Writes the
// k selected indices, ascending, to out_idx and their scores to out_val
// (nullable); both may point to global memory or LDS.  With have_range the
// caller passes the row's exact minimum and maximum (saves one pass).
template <int NT, int KREG, typename Load>
__device__ __forceinline__ void block_select(Load load_score, int S, int k, int32_t* out_idx,
                                             float* out_val, SelectSmem<NT / 64>& sm,
                                             bool have_range = false, float lo_in = 0.f,
                                             float hi_in = 0.f) {
  constexpr int NW = NT / 64;
  constexpr int PER_WAVE = KREG * 64;  // contiguous indices owned by one wave
  constexpr int BPL = kBins / NW / 64;  // bins per lane in the scan
  static_assert(BPL >= 1 && kBins % (NW * 64) == 0, "bins split over the waves");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // element j of this thread has index wave*per_wave + j*64 + lane: each wave
  // owns a contiguous range of per_wave indices (KREG*64 with registers)
  constexpr int NJ = KREG > 0 ? KREG : 1;
  const int per_wave = KREG > 0 ? PER_WAVE : (S + NW * 64 - 1) / (NW * 64) * 64;
  const int nj = per_wave / 64;
  auto index_of = [&](int j) -> int { return wave * per_wave + j * 64 + lane; };
  float sv[NJ];
  if constexpr (KREG > 0) {
#pragma unroll
    for (int j = 0; j < KREG; j++) sv[j] = load_score(index_of(j));
  }
  // f(j, i, v) for every element of this thread (i may be >= S)
  auto each = [&](auto&& f) {
    if constexpr (KREG > 0) {
#pragma unroll
      for (int j = 0; j < KREG; j++) f(j, index_of(j), sv[j]);
    } else {
      for (int j = 0; j < nj; j++) {
        const int i = index_of(j);
        f(j, i, load_score(i));
      }
    }
  };

  // ---- range of the row
  for (int e = tid; e < kBins; e += NT) sm.hist[e] = 0u;
  if (tid == 0) sm.n_cand = 0;
  float lo = lo_in, hi = hi_in;
  if (!have_range) {
    lo = INFINITY;
    hi = -INFINITY;
    each([&](int, int i, float v) {
      if (i < S) {
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
      }
    });
    lo = -wave_max(-lo);
    hi = wave_max(hi);
    if (lane == 0) {
      sm.wmin[wave] = lo;
      sm.wmax[wave] = hi;
    }
  }
  __syncthreads();
  if (!have_range) {
    lo = sm.wmin[0];
    hi = sm.wmax[0];
#pragma unroll
    for (int w = 1; w < NW; w++) {
      lo = fminf(lo, sm.wmin[w]);
      hi = fmaxf(hi, sm.wmax[w]);
    }
  }
  const float range = hi - lo;
  float scale = (range > 0.f && range < INFINITY) ? (float)(kBins - 1) / range : 0.f;
  if (!(scale < INFINITY)) scale = 0.f;  // subnormal range: everything in one bin

  // ---- 1. linear-bin histogram and the bin of the k-th largest score
  each([&](int, int i, float v) {
    if (i < S) atomicAdd(&sm.hist[lin_bin(v, lo, scale)], 1u);
  });
  __syncthreads();
  // descending scan: wave w covers positions [w*kBins/NW, (w+1)*kBins/NW),
  // position q holds bin kBins-1-q, each lane BPL consecutive positions
  unsigned c[BPL];
  unsigned tot = 0u;
#pragma unroll
  for (int u = 0; u < BPL; u++) {
    c[u] = sm.hist[kBins - 1 - (wave * (kBins / NW) + lane * BPL + u)];
    tot += c[u];
  }
  const unsigned incl = wave_incl_scan(tot);
  if (lane == 63) sm.wtot[wave] = incl;
  __syncthreads();
  unsigned before = incl - tot;
  for (int w = 0; w < wave; w++) before += sm.wtot[w];
#pragma unroll
  for (int u = 0; u < BPL; u++) {
    const unsigned after = before + c[u];
    if (before < (unsigned)k && after >= (unsigned)k) {  // exactly one position
      sm.sel_bin = kBins - 1 - (wave * (kBins / NW) + lane * BPL + u);
      sm.sel_gt = (int)before;
      sm.sel_eq = (int)c[u];
    }
    before = after;
  }
  __syncthreads();
  const int bstar = sm.sel_bin;
  const int rem = k - sm.sel_gt;  // 1 <= rem <= members of b*
  const int nb = sm.sel_eq;

  // ---- 2. exact threshold key inside b*
  if (nb <= kFewCandidates) {
    each([&](int, int i, float v) {
      if (i < S && lin_bin(v, lo, scale) == bstar) {
        const int slot = atomicAdd(&sm.n_cand, 1);
        sm.cand_key[slot] = order_key(v);
        sm.cand_idx[slot] = i;
      }
    });
    __syncthreads();
    if (wave == 0) {
      const bool mine = lane < nb;
      const unsigned mk = mine ? sm.cand_key[lane] : 0u;
      const int mi = mine ? sm.cand_idx[lane] : INT_MAX;
      int rank = 0;
      for (int m = 0; m < nb; m++) {
        const unsigned ok = sm.cand_key[m];
        const int oi = sm.cand_idx[m];
        rank += (ok > mk || (ok == mk && oi < mi)) ? 1 : 0;
      }
      const unsigned long long at = __ballot(mine && rank == rem - 1);  // one lane
      const int src = at ? __ffsll((long long)at) - 1 : 0;
      const unsigned T = (unsigned)__shfl((int)mk, src, 64);
      const unsigned long long teq = __ballot(mine && mk == T && rank < rem);
      if (lane == 0) {
        sm.thr_key = T;
        sm.thr_take = __popcll(teq);
      }
    }
  } else {
    unsigned prefix = 0u, pmask = 0u;
    int rr = rem;
    for (int pass = 0; pass < 4; pass++) {
      const int shift = 24 - 8 * pass;
      for (int e = tid; e < NW * 256; e += NT) (&sm.whist[0][0])[e] = 0u;
      __syncthreads();
      each([&](int, int i, float v) {
        if (i < S && lin_bin(v, lo, scale) == bstar) {
          const unsigned key = order_key(v);
          if ((key & pmask) == prefix) atomicAdd(&sm.whist[wave][(key >> shift) & 0xffu], 1u);
        }
      });
      __syncthreads();
      if (wave == 0) {
        unsigned cc[4];
        unsigned t4 = 0u;
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const int dg = 255 - (lane * 4 + u);
          unsigned s = 0u;
#pragma unroll
          for (int w = 0; w < NW; w++) s += sm.whist[w][dg];
          cc[u] = s;
          t4 += s;
        }
        unsigned bf = wave_incl_scan(t4) - t4;
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const unsigned af = bf + cc[u];
          if (bf < (unsigned)rr && af >= (unsigned)rr) {
            sm.r_digit = 255u - (unsigned)(lane * 4 + u);
            sm.r_gt = bf;
            sm.r_eq = cc[u];
          }
          bf = af;
        }
      }
      __syncthreads();
      rr -= (int)sm.r_gt;
      prefix |= sm.r_digit << shift;
      pmask |= 0xffu << shift;
      const bool done = (int)sm.r_eq == rr;  // the whole prefix group is taken
      __syncthreads();
      if (done) break;
    }
    // T = smallest key of the taken prefix group: everything >= T is selected
    unsigned tmin = 0xffffffffu;
    each([&](int, int i, float v) {
      if (i < S && lin_bin(v, lo, scale) == bstar) {
        const unsigned key = order_key(v);
        if ((key & pmask) == prefix) tmin = min(tmin, key);
      }
    });
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) tmin = min(tmin, (unsigned)__shfl_xor((int)tmin, o, 64));
    if (lane == 0) sm.wtot[wave] = tmin;
    __syncthreads();
    if (tid == 0) {
      unsigned t = sm.wtot[0];
      for (int w = 1; w < NW; w++) t = min(t, sm.wtot[w]);
      sm.thr_key = t;
      // all passes resolved: take rr of the keys equal to T; early stop: all of them
      sm.thr_take = (pmask == 0xffffffffu) ? rr : INT_MAX;
    }
  }
  __syncthreads();

  // ---- 3. ordered compaction
  const unsigned T = sm.thr_key;
  const int r = sm.thr_take;
  int32_t* irow = out_idx;
  float* vrow = out_val;
  int gt_w = 0, eq_w = 0;
  each([&](int, int i, float v) {
    const unsigned key = order_key(v);
    gt_w += __popcll(__ballot(i < S && key > T));
    eq_w += __popcll(__ballot(i < S && key == T));
  });
  if (lane == 0) {
    sm.wcnt[wave][0] = gt_w;
    sm.wcnt[wave][1] = eq_w;
  }
  __syncthreads();
  int out = 0, eq_seen = 0;
  for (int w = 0; w < wave; w++) {
    const int ce = sm.wcnt[w][1];
    const int take = max(0, min(ce, r - eq_seen));
    out += sm.wcnt[w][0] + take;
    eq_seen += ce;
  }
  each([&](int, int i, float v) {
    const unsigned key = order_key(v);
    const bool gt = i < S && key > T, eq = i < S && key == T;
    const unsigned long long be = __ballot(eq);
    const bool sel = gt || (eq && eq_seen + lane_rank(be) < r);
    const unsigned long long bs = __ballot(sel);
    const int pos = out + lane_rank(bs);
    if (sel && pos < k) {  // exactly k are selected; the bound only guards the row
      irow[pos] = i;
      if (vrow) vrow[pos] = v;
    }
    out += __popcll(bs);
    eq_seen += __popcll(be);
  });
}

}  // namespace loki
