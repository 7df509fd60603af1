// Block-wide exact top-k selection (device code shared by the stand-alone
// top-k kernel and the fused decode kernel).
//
// Loki (briefgpt.xyz abstract; poster page "TL;DR" and Figure 1 right): the
// tokens of the KV-cache are ranked by their low-dimensional scores and only
// the top k are kept for the exact attention.
//
// Exact selection of the k elements of a row of S scores that rank first by
// (score descending, index ascending); the indices come out ascending.
//  1. Linear binning.  bin(s) = clamp(floor((s - lo) * scale), 0, 2047) is a
//     non-decreasing function of s for ANY lo and scale >= 0, so every score
//     in a higher bin exceeds every score in a lower one.  One LDS histogram
//     of 2048 bins (few atomic collisions on spread data) and a DPP prefix
//     scan over the bins in descending order give the bin b* that holds the
//     k-th largest score.  lo and scale come from the row's range or, in the
//     fused kernel, from a first batch of scores (the histogram is then built
//     while scoring; clamping keeps the binning monotone).
//  2. The last taken element.  Elements are ordered by (order-preserving key
//     descending, index ascending); the k-th one, (T, I), is found inside b*:
//     with few members (the common case) one pass over the row collects them
//     and counts, per wave, the members of higher bins, then a candidate's
//     rank is one ballot over all candidates (the waves take the candidates
//     in turn; the fused kernel's select_rows ranks its few in one wave);
//     otherwise radix passes over 8-bit digits
//     of the members' keys (per-wave LDS histograms), then the position of the
//     last taken key among equal keys, then a counting pass.
//  3. Ordered compaction: element i is taken iff key > T or (key == T and
//     i <= I).  Each wave owns a contiguous index range whose taken count is
//     known from step 2; each wave writes its indices at offsets from mbcnt
//     ranks of its ballots.
// Order keys stay in registers when S <= threads * KREG, else the scores are
// re-read; padding elements (index >= S) are masked in every ballot.
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

// Inverse of order_key (a -0 score comes back as +0).
__device__ __forceinline__ float key_score(unsigned key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

__device__ __forceinline__ int lin_bin(float s, float lo, float scale) {
  const int b = (int)((s - lo) * scale);
  return b < 0 ? 0 : (b > kBins - 1 ? kBins - 1 : b);
}

// scale of the linear binning of [lo, hi]; 0 (one bin) when the range is empty,
// not finite or too small to scale
__device__ __forceinline__ float bin_scale(float lo, float hi) {
  const float range = hi - lo;
  float scale = (range > 0.f && range < INFINITY) ? (float)(kBins - 1) / range : 0.f;
  return scale < INFINITY ? scale : 0.f;
}

// LDS scratch of one selection.
template <int NW>
struct SelectSmem {
  unsigned hist[kBins];
  unsigned whist[NW][256];
  float wmin[NW], wmax[NW];
  float wsum[NW], wsq[NW];
  unsigned wtot[NW];
  int sel_bin, sel_gt, sel_eq, n_cand;
  unsigned cand_key[kFewCandidates];
  int cand_idx[kFewCandidates];
  unsigned thr_key, r_digit, r_gt, r_eq;
  int thr_idx;
  int wcnt[NW];
};

// Zero the histogram (all NT threads; a barrier must follow before use).
template <int NT, int NW>
__device__ __forceinline__ void select_clear(SelectSmem<NW>& sm) {
  for (int e = threadIdx.x; e < kBins; e += NT) sm.hist[e] = 0u;
  if (threadIdx.x == 0) sm.n_cand = 0;
}

// A thread's share of a row of S scores, as order keys: element j has index
// wave*per_wave + j*64 + lane, so each wave owns a contiguous index range.
// With KREG > 0 (S <= NT*KREG) the keys are computed once and kept in
// registers; otherwise (KREG == 0) each pass re-reads the scores through
// load_score.  load_score(i) returns score i for i < S and any value for
// i >= S: every use masks those elements with i < S.
template <int NT, int KREG, typename Load>
struct RowView {
  static constexpr int NW = NT / 64;
  static constexpr int NJ = KREG > 0 ? KREG : 1;
  Load load_score;
  int S, per_wave, nj, base;
  unsigned kv[NJ];

  __device__ __forceinline__ RowView(Load l, int S_) : load_score(l), S(S_) {
    per_wave = KREG > 0 ? KREG * 64 : (S + NW * 64 - 1) / (NW * 64) * 64;
    nj = per_wave / 64;
    base = (threadIdx.x >> 6) * per_wave + (threadIdx.x & 63);
    if constexpr (KREG > 0) {
#pragma unroll
      for (int j = 0; j < KREG; j++) kv[j] = order_key(load_score(base + j * 64));
    }
  }

  // f(i, key) for each element of this thread (i may be >= S)
  template <typename F>
  __device__ __forceinline__ void each(F&& f) {
    if constexpr (KREG > 0) {
#pragma unroll
      for (int j = 0; j < KREG; j++) f(base + j * 64, kv[j]);
    } else {
      for (int j = 0; j < nj; j++) {
        const int i = base + j * 64;
        f(i, order_key(load_score(i)));
      }
    }
  }
};

// Step 1b: descending scan over the histogram; sets sm.sel_bin (the bin b*
// holding the k-th largest score), sm.sel_gt (members of higher bins) and
// sm.sel_eq (members of b*).  All NT threads; ends with a barrier.
template <int NT>
__device__ __forceinline__ void select_scan(SelectSmem<NT / 64>& sm, int k) {
  constexpr int NW = NT / 64;
  constexpr int BPL = kBins / NW / 64;  // bins per lane in the scan
  static_assert(BPL >= 1 && kBins % (NW * 64) == 0, "bins split over the waves");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // wave w covers positions [w*kBins/NW, (w+1)*kBins/NW), position q holds bin kBins-1-q
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
}

// Step 2 for a crowded b*: radix passes over 8-bit digits of the keys of
// b*'s members (per-wave LDS histograms) give (T, I), the last taken element,
// in sm.thr_key / sm.thr_idx.  All NT threads; ends with a barrier.
template <int NT, int KREG, typename Load>
__device__ __forceinline__ void radix_threshold(RowView<NT, KREG, Load>& row, int bstar, int rem,
                                                float lo, float scale, SelectSmem<NT / 64>& sm) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = row.S;
  // radix passes over the keys of b*'s members
  unsigned prefix = 0u, pmask = 0u;
  int rr = rem;
  bool whole = false;
  for (int pass = 0; pass < 4; pass++) {
    const int shift = 24 - 8 * pass;
    for (int e = tid; e < NW * 256; e += NT) (&sm.whist[0][0])[e] = 0u;
    __syncthreads();
    row.each([&](int i, unsigned key) {
      if (i < S && lin_bin(key_score(key), lo, scale) == bstar && (key & pmask) == prefix)
        atomicAdd(&sm.whist[wave][(key >> shift) & 0xffu], 1u);
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
    whole = (int)sm.r_eq == rr;  // the whole prefix group is taken
    __syncthreads();
    if (whole) break;
  }
  // T: the smallest key of the taken prefix group (the exact key when all
  // passes ran); I: every key equal to T is taken if the group was taken
  // whole, else the rr-th one in index order
  unsigned tmin = 0xffffffffu;
  row.each([&](int i, unsigned key) {
    if (i < S && lin_bin(key_score(key), lo, scale) == bstar && (key & pmask) == prefix)
      tmin = min(tmin, key);
  });
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) tmin = min(tmin, (unsigned)__shfl_xor((int)tmin, o, 64));
  if (lane == 0) sm.wtot[wave] = tmin;
  __syncthreads();
  unsigned T = sm.wtot[0];
  for (int w = 1; w < NW; w++) T = min(T, sm.wtot[w]);
  if (whole) {
    if (tid == 0) {
      sm.thr_key = T;
      sm.thr_idx = INT_MAX;
    }
  } else {
    // the rr-th index (ascending) among keys equal to T
    int cnt = 0;
    row.each([&](int i, unsigned key) { cnt += __popcll(__ballot(i < S && key == T)); });
    if (lane == 0) sm.wcnt[wave] = cnt;
    __syncthreads();
    int seen = 0;
    for (int w = 0; w < wave; w++) seen += sm.wcnt[w];
    row.each([&](int i, unsigned key) {
      const bool eq = i < S && key == T;
      const unsigned long long be = __ballot(eq);
      if (eq && seen + lane_rank(be) == rr - 1) {
        sm.thr_key = T;
        sm.thr_idx = i;
      }
      seen += __popcll(be);
    });
  }
  __syncthreads();
}

// Steps 1 (after the histogram) to 3.  sm.hist holds the histogram of the
// row under (lo, scale) and sm.n_cand is 0.  All NT threads call it together.
template <int NT, int KREG, typename Load>
__device__ __forceinline__ void select_from_histogram(RowView<NT, KREG, Load>& row, int k,
                                                      int32_t* out_idx, float* out_val,
                                                      SelectSmem<NT / 64>& sm, float lo,
                                                      float scale) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = row.S;

  select_scan<NT>(sm, k);
  const int bstar = sm.sel_bin;
  const int rem0 = k - sm.sel_gt;  // 1 <= rem0 <= members of b*
  int rem = rem0, nb = sm.sel_eq;

  // ---- 1c. a crowded b* (a wide score range, e.g. a few large outliers,
  // squeezes the bulk into few bins): split b*'s interval linearly into kBins
  // sub-bins -- monotone in the score, so the order is kept -- and find the
  // sub-bin holding the rem-th largest member.  sub < 0: not refined.
  int sub = -1;
  float lo2 = 0.f, scale2 = 0.f;
  if (nb > kFewCandidates && scale > 0.f && scale * (float)kBins < INFINITY) {
    lo2 = lo + (float)bstar / scale;
    scale2 = scale * (float)kBins;
    for (int e = tid; e < kBins; e += NT) sm.hist[e] = 0u;
    __syncthreads();  // every thread has read the first scan's results
    row.each([&](int i, unsigned key) {
      const float sc = key_score(key);
      if (i < S && lin_bin(sc, lo, scale) == bstar) atomicAdd(&sm.hist[lin_bin(sc, lo2, scale2)], 1u);
    });
    __syncthreads();
    select_scan<NT>(sm, rem0);
    sub = sm.sel_bin;
    rem = rem0 - sm.sel_gt;
    nb = sm.sel_eq;
  }
  // position of a key against the threshold group: 1 above, 0 inside, -1 below
  auto side = [&](unsigned key) -> int {
    const float sc = key_score(key);
    const int bn = lin_bin(sc, lo, scale);
    if (bn != bstar) return bn > bstar ? 1 : -1;
    if (sub < 0) return 0;
    const int sb = lin_bin(sc, lo2, scale2);
    return sb > sub ? 1 : (sb == sub ? 0 : -1);
  };

  // ---- 2. the last taken element (T, I) inside the threshold group, and the
  // number of taken elements of each wave's index range in sm.wcnt
  if (nb <= kFewCandidates) {
    // one pass: members of the group become candidates, members above it are
    // counted per wave
    unsigned gt = 0u;
    auto visit = [&](int i, unsigned key, int sd) {
      const bool valid = i < S;
      gt += (unsigned)__popcll(__ballot(valid && sd > 0));
      const bool cand = valid && sd == 0;
      if (__ballot(cand) != 0ull) {  // rare: this wave row holds members of the group
        if (cand) {
          const int slot = atomicAdd(&sm.n_cand, 1);
          sm.cand_key[slot] = key;
          sm.cand_idx[slot] = i;
        }
      }
    };
    if (sub < 0) {
      row.each([&](int i, unsigned key) {
        const int bn = lin_bin(key_score(key), lo, scale);
        visit(i, key, bn > bstar ? 1 : (bn == bstar ? 0 : -1));
      });
    } else {
      row.each([&](int i, unsigned key) { visit(i, key, side(key)); });
    }
    if (lane == 0) sm.wcnt[wave] = (int)gt;
    __syncthreads();
    // rank of candidate c = members ordered before it by (key descending,
    // index ascending): one ballot over the candidates on the lanes; the
    // waves take the candidates in turn
    {
      const bool mine = lane < nb;
      const unsigned mk = mine ? sm.cand_key[lane] : 0u;
      const int mi = mine ? sm.cand_idx[lane] : INT_MAX;
      for (int c = wave; c < nb; c += NW) {
        const unsigned ck = (unsigned)__builtin_amdgcn_readlane((int)mk, c);
        const int ci = __builtin_amdgcn_readlane(mi, c);
        const int rank = __popcll(__ballot(mine && (mk > ck || (mk == ck && mi < ci))));
        if (lane == 0) {
          if (rank == rem - 1) {  // exactly one candidate
            sm.thr_key = ck;
            sm.thr_idx = ci;
          }
          if (rank < rem) atomicAdd(&sm.wcnt[ci / row.per_wave], 1);
        }
      }
    }
    __syncthreads();
  } else {
    radix_threshold<NT, KREG>(row, bstar, rem0, lo, scale, sm);
    const unsigned Tk = sm.thr_key;
    const int Ik = sm.thr_idx;
    int cnt = 0;
    row.each([&](int i, unsigned key) {
      cnt += __popcll(__ballot(i < S && (key > Tk || (key == Tk && i <= Ik))));
    });
    if (lane == 0) sm.wcnt[wave] = cnt;
    __syncthreads();
  }

  // ---- 3. ordered compaction: take key > T, or key == T with index <= I
  const unsigned T = sm.thr_key;
  const int I = sm.thr_idx;
  int out = 0;
  for (int w = 0; w < wave; w++) out += sm.wcnt[w];
  row.each([&](int i, unsigned key) {
    const bool sel = i < S && (key > T || (key == T && i <= I));
    const unsigned long long bs = __ballot(sel);
    const int pos = out + lane_rank(bs);
    if (sel && pos < k) {  // exactly k are taken; the bound only guards the row
      out_idx[pos] = i;
      if (out_val) out_val[pos] = key_score(key);
    }
    out += __popcll(bs);
  });
}

// Entries of each wave's list in select_rows: the lists fill sm.hist and
// sm.whist, which lie back to back (the scan is done with the first, the
// radix passes start on the second only after the lists are copied out).
template <int NT>
constexpr int kRowListCap = kBins / (NT / 64) + 256;

// Selection for a caller that attends over the selected rows right away.
// Rows [0, sel_gt) are the members of the bins above b*, in index order: one
// pass appends them to per-wave lists kept in sm.hist / sm.whist (the scan
// no longer needs them) while it collects b*'s members; rows [sel_gt, k) are
// the taken members of b*, also in index order.  mid() runs between that
// pass and the barrier after it.  Writes rows_idx / rows_val (score, -0 as
// +0) [0, k) and sm.sel_gt; the caller needs a barrier before reading them.
// Requires that no wave's list outgrows kRowListCap<NT>: a list holds fewer
// than k entries and at most a wave's share of the row (KREG * 64), so
// k - 1 <= kRowListCap<NT> or KREG * 64 <= kRowListCap<NT> suffices.
template <int NT, int KREG, typename Load, typename Mid>
__device__ __forceinline__ void select_rows(RowView<NT, KREG, Load>& row, int k, int32_t* rows_idx,
                                            float* rows_val, SelectSmem<NT / 64>& sm, float lo,
                                            float scale, Mid&& mid) {
  constexpr int NW = NT / 64;
  constexpr int CAP = kRowListCap<NT>;  // >= the length of any wave's list
  static_assert(sizeof(SelectSmem<NW>::hist) + sizeof(SelectSmem<NW>::whist) >=
                    sizeof(int) * (size_t)NW * CAP, "lists fit hist and whist");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = row.S;

  select_scan<NT>(sm, k);
  const int bstar = sm.sel_bin, sel_gt = sm.sel_gt, rem = k - sel_gt, nb = sm.sel_eq;
  const bool few = nb <= kFewCandidates;
  int* lists = reinterpret_cast<int*>(sm.hist);

  int cnt = 0;
  row.each([&](int i, unsigned key) {
    const int bn = lin_bin(key_score(key), lo, scale);
    const bool valid = i < S;
    const bool sure = valid && bn > bstar;
    const unsigned long long bs = __ballot(sure);
    if (sure) lists[wave * CAP + cnt + lane_rank(bs)] = i;
    cnt += __popcll(bs);
    const bool cand = few && valid && bn == bstar;
    if (__ballot(cand) != 0ull) {  // rare: this wave row holds members of b*
      if (cand) {
        const int slot = atomicAdd(&sm.n_cand, 1);
        sm.cand_key[slot] = key;
        sm.cand_idx[slot] = i;
      }
    }
  });
  if (lane == 0) sm.wcnt[wave] = cnt;
  mid();
  __syncthreads();

  // rows [0, sel_gt): the per-wave lists back to back
  int pre[NW];
  pre[0] = 0;
#pragma unroll
  for (int w = 1; w < NW; w++) pre[w] = pre[w - 1] + sm.wcnt[w - 1];
  for (int r = tid; r < sel_gt; r += NT) {
    int w = 0;
#pragma unroll
    for (int v = 1; v < NW; v++) w += r >= pre[v] ? 1 : 0;
    const int i = lists[w * CAP + r - pre[w]];
    rows_idx[r] = i;
    rows_val[r] = key_score(order_key(row.load_score(i)));
  }

  // rows [sel_gt, k): the taken members of b*
  if (few) {
    if (wave == 0) {
      // candidate m on lane m; rank = members ordered before it by
      // (key descending, index ascending); the rem first are taken
      const bool mine = lane < nb;
      const unsigned mk = mine ? sm.cand_key[lane] : 0u;
      const int mi = mine ? sm.cand_idx[lane] : INT_MAX;
      int rank = 0;
      for (int m = 0; m < nb; m++) {
        const unsigned ok = (unsigned)__builtin_amdgcn_readlane((int)mk, m);
        const int oi = __builtin_amdgcn_readlane(mi, m);
        rank += (ok > mk || (ok == mk && oi < mi)) ? 1 : 0;
      }
      const bool taken = mine && rank < rem;
      int pos = 0;  // among the taken, by index
      for (int m = 0; m < nb; m++) {
        const int orank = __builtin_amdgcn_readlane(rank, m);
        const int oi = __builtin_amdgcn_readlane(mi, m);
        pos += (orank < rem && oi < mi) ? 1 : 0;
      }
      if (taken) {
        rows_idx[sel_gt + pos] = mi;
        rows_val[sel_gt + pos] = key_score(mk);
      }
    }
  } else {
    __syncthreads();  // every list entry is copied out before whist is reused
    radix_threshold<NT, KREG>(row, bstar, rem, lo, scale, sm);
    const unsigned T = sm.thr_key;
    const int I = sm.thr_idx;
    auto taken = [&](int i, unsigned key) -> bool {
      return i < S && lin_bin(key_score(key), lo, scale) == bstar &&
             (key > T || (key == T && i <= I));
    };
    int c2 = 0;
    row.each([&](int i, unsigned key) { c2 += __popcll(__ballot(taken(i, key))); });
    if (lane == 0) sm.wcnt[wave] = c2;
    __syncthreads();
    int out = sel_gt;
    for (int w = 0; w < wave; w++) out += sm.wcnt[w];
    row.each([&](int i, unsigned key) {
      const bool t = taken(i, key);
      const unsigned long long bt = __ballot(t);
      const int pos = out + lane_rank(bt);
      if (t && pos < k) {
        rows_idx[pos] = i;
        rows_val[pos] = key_score(key);
      }
      out += __popcll(bt);
    });
  }
}

// The rows of select_rows in ascending index order, to global memory: the two
// index-ordered parts [0, n1) (the members of bins above b*) and [n1, k) (the
// taken members of b*, usually few) merged: a row of the first part moves up
// by the taken members below it, a taken member by the first-part rows below
// it (binary search).  All NT threads, after the rows are visible.
__device__ __forceinline__ void write_rows_in_index_order(const int32_t* rows, int n1, int k,
                                                          int32_t* out, int NT) {
  const int n2 = k - n1;
  for (int r = threadIdx.x; r < k; r += NT) {
    const int t = rows[r];
    int pos;
    if (r < n1) {
      pos = r;
      for (int j = 0; j < n2; j++) pos += rows[n1 + j] < t ? 1 : 0;  // broadcast reads
    } else {
      int lo = 0, hi = n1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (rows[mid] < t) lo = mid + 1; else hi = mid;
      }
      pos = (r - n1) + lo;
    }
    out[pos] = t;
  }
}

// Rows of more than 16384 scores (32 order keys per thread, or re-read
// scores): a bin of the linear binning holds 8 or more scores on average, and
// a few large outliers that stretch [min, max] crowd the bin of the k-th
// score; these rows bin over mean +- 6 sd instead.  Shorter rows keep
// [min, max] (the moments cost more there than the rare refinement).
template <int KREG>
constexpr bool kClampRange = KREG == 0 || KREG >= 32;

// Whole selection from the scores alone (range, histogram, steps 1-3).
// With have_range the caller passes the row's minimum and maximum.
template <int NT, int KREG, typename Load>
__device__ __forceinline__ void block_select(Load load_score, int S, int k, int32_t* out_idx,
                                             float* out_val, SelectSmem<NT / 64>& sm,
                                             bool have_range = false, float lo_in = 0.f,
                                             float hi_in = 0.f) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  RowView<NT, KREG, Load> row(load_score, S);
  select_clear<NT>(sm);
  float lo = lo_in, hi = hi_in;
  if (!have_range) {
    // the range through the keys (integer min / max) and, for long rows,
    // the first two moments of the scores; padding excluded
    unsigned kmin = 0xffffffffu, kmax = 0u;
    float sum = 0.f, sq = 0.f;
    row.each([&](int i, unsigned key) {
      const bool valid = i < S;
      kmin = min(kmin, valid ? key : 0xffffffffu);
      kmax = max(kmax, valid ? key : 0u);
      if constexpr (kClampRange<KREG>) {
        // the empty asm keeps the compiler from holding these scores in
        // registers for the histogram pass, which recomputes them
        unsigned kk = key;
        asm volatile("" : "+v"(kk));
        const float v = valid ? key_score(kk) : 0.f;
        sum += v;
        sq = fmaf(v, v, sq);
      }
    });
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      kmin = min(kmin, (unsigned)__shfl_xor((int)kmin, o, 64));
      kmax = max(kmax, (unsigned)__shfl_xor((int)kmax, o, 64));
    }
    if constexpr (kClampRange<KREG>) {
      sum = wave_sum(sum);
      sq = wave_sum(sq);
    }
    if (lane == 0) {
      sm.wmin[wave] = key_score(kmin);
      sm.wmax[wave] = key_score(kmax);
      sm.wsum[wave] = sum;
      sm.wsq[wave] = sq;
    }
  }
  __syncthreads();
  if (!have_range) {
    lo = sm.wmin[0];
    hi = sm.wmax[0];
    float sum = sm.wsum[0], sq = sm.wsq[0];
#pragma unroll
    for (int w = 1; w < NW; w++) {
      lo = fminf(lo, sm.wmin[w]);
      hi = fmaxf(hi, sm.wmax[w]);
      sum += sm.wsum[w];
      sq += sm.wsq[w];
    }
    if constexpr (kClampRange<KREG>) {
      // bin over [mean - 6 sd, mean + 6 sd] within [min, max]: a few large
      // outliers then no longer squeeze the bulk into few bins (scores
      // outside land in the end bins, and clamped linear bins stay
      // monotone).  A non-finite mean or spread leaves the range as it is
      // (fmaxf / fminf return the non-NaN operand).
      const float mean = sum / (float)S;
      const float sd = sqrtf(fmaxf(sq / (float)S - mean * mean, 0.f));
      lo = fmaxf(lo, mean - 6.f * sd);
      hi = fminf(hi, mean + 6.f * sd);
    }
  }
  const float scale = bin_scale(lo, hi);
  row.each([&](int i, unsigned key) {
    if (i < S) atomicAdd(&sm.hist[lin_bin(key_score(key), lo, scale)], 1u);
  });
  __syncthreads();
  select_from_histogram<NT, KREG>(row, k, out_idx, out_val, sm, lo, scale);
}

}  // namespace loki
