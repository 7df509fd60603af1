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
//     one-launch kernels, from a first batch of scores (the histogram is then
//     built while scoring; clamping keeps the binning monotone).
//  2. The last taken element.  Elements are ordered by (order-preserving key
//     descending, index ascending); the k-th one, (T, I), is found inside b*:
//     with few members (the common case) one pass over the row collects them
//     and counts, per wave, the members of higher bins, then a candidate's
//     rank is one ballot over all candidates (the waves take the candidates
//     in turn); otherwise radix passes over 8-bit digits
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

__host__ __device__ __forceinline__ unsigned order_key(float s) {
  unsigned u = __builtin_bit_cast(unsigned, s);
  if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// order_key for a score that is not -0 (the caller adds +0, which turns -0
// into +0 and leaves every other value as it is): three instructions.
__host__ __device__ __forceinline__ unsigned order_key_nz(float s) {
  const unsigned u = __builtin_bit_cast(unsigned, s);
  return u ^ ((unsigned)((int)u >> 31) | 0x80000000u);
}

// Inverse of order_key (a -0 score comes back as +0).
__host__ __device__ __forceinline__ float key_score(unsigned key) {
  return __builtin_bit_cast(float, (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Linear bin of score s: floor((s - lo) * scale) clamped to [0, kBins - 1].
// The clamping is done in float, before the conversion to int, so the bin is
// defined for every s, lo and scale, and it never decreases as order_key(s)
// grows: a product at or above kBins - 1 (+inf included) takes the top bin,
// one at or below 0 (-inf included) bin 0; scale 0 puts every score in bin 0;
// a NaN score goes where its order key ranks it: the top bin when its sign
// bit is clear (above +inf), bin 0 when it is set (below -inf).
__host__ __device__ __forceinline__ int lin_bin(float s, float lo, float scale) {
  const float x = (s - lo) * scale;
  const int b = (int)fminf(fmaxf(x, 0.f), (float)(kBins - 1));  // fmaxf(NaN, 0) is 0
  if (x == x || scale == 0.f) return b;
  return (__builtin_bit_cast(unsigned, s) & 0x80000000u) ? 0 : kBins - 1;
}

// scale of the linear binning of [lo, hi]; 0 (one bin) when the range is empty,
// not finite or too small to scale
__host__ __device__ __forceinline__ float bin_scale(float lo, float hi) {
  const float range = hi - lo;
  float scale = (range > 0.f && range < INFINITY) ? (float)(kBins - 1) / range : 0.f;
  return scale < INFINITY ? scale : 0.f;
}

// LDS scratch of one selection, with the radix passes' per-wave histograms
// (whist) right after the bin histogram.
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
  unsigned key_lo, key_hi1;  // keys of the threshold group: [key_lo, key_hi1]
};

// The same without whist: for callers that put the per-wave histograms of the
// radix passes (NW x 256 words, used only after the bin histogram's scans) in
// LDS they reuse, and pass them to select_from_histogram.
template <int NW>
struct SelectSmemLite {
  unsigned hist[kBins];
  float wmin[NW], wmax[NW];
  float wsum[NW], wsq[NW];
  unsigned wtot[NW];
  int sel_bin, sel_gt, sel_eq, n_cand;
  unsigned cand_key[kFewCandidates];
  int cand_idx[kFewCandidates];
  unsigned thr_key, r_digit, r_gt, r_eq;
  int thr_idx;
  int wcnt[NW];
  unsigned key_lo, key_hi1;  // keys of the threshold group: [key_lo, key_hi1]
};

// Zero the histogram (all NT threads; a barrier must follow before use).
template <int NT, typename SM>
__device__ __forceinline__ void select_clear(SM& sm) {
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

// A thread's share of a row of S order keys held in LDS (element j of the
// thread: index wave*KREG*64 + j*64 + lane, as RowView), kept in registers;
// elements past the row get key 0.  keys[i] is read for i < S only.
template <int NT, int KREG>
struct KeyRow {
  static_assert(KREG > 0, "keys in registers");
  int S, per_wave, base;
  unsigned kv[KREG];

  __device__ __forceinline__ KeyRow(const unsigned* keys, int S_) : S(S_) {
    per_wave = KREG * 64;
    base = (threadIdx.x >> 6) * per_wave + (threadIdx.x & 63);
    if (S >= NT * KREG) {  // a full row: no element to check
#pragma unroll
      for (int j = 0; j < KREG; j++) kv[j] = keys[base + j * 64];
    } else {
#pragma unroll
      for (int j = 0; j < KREG; j++) {
        const int i = base + j * 64;
        kv[j] = i < S ? keys[i] : 0u;
      }
    }
  }

  template <typename F>
  __device__ __forceinline__ void each(F&& f) {
#pragma unroll
    for (int j = 0; j < KREG; j++) f(base + j * 64, kv[j]);
  }
};

// Step 1b: descending scan over the histogram; sets sm.sel_bin (the bin b*
// holding the k-th largest score), sm.sel_gt (members of higher bins) and
// sm.sel_eq (members of b*).  All NT threads; ends with a barrier.
template <int NT, typename SM>
__device__ __forceinline__ void select_scan(SM& sm, int k) {
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

// Step 2 for a crowded threshold group: radix passes over 8-bit digits of the
// keys of the group's members (member(key) true; per-wave LDS histograms) give
// (T, I), the rem-th member in the selection order, in sm.thr_key /
// sm.thr_idx; whist: NT/64 rows of 256 words of LDS.  All NT threads; ends
// with a barrier.
// PADDED: member() is false for every padding element (index >= S), so the
// index is not checked.
template <int NT, int KREG, bool PADDED = false, typename Row, typename SM, typename Member>
__device__ __forceinline__ void radix_threshold_of(Row& row, Member&& member,
                                                   int rem, SM& sm, unsigned (*whist)[256]) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = row.S;
  // radix passes over the keys of b*'s members
  unsigned prefix = 0u, pmask = 0u;
  int rr = rem;
  bool whole = false;
  for (int pass = 0; pass < 4; pass++) {
    const int shift = 24 - 8 * pass;
    for (int e = tid; e < NW * 256; e += NT) (&whist[0][0])[e] = 0u;
    __syncthreads();
    row.each([&](int i, unsigned key) {
      if ((PADDED || i < S) && member(key) && (key & pmask) == prefix)
        atomicAdd(&whist[wave][(key >> shift) & 0xffu], 1u);
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
        for (int w = 0; w < NW; w++) s += whist[w][dg];
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
    if ((PADDED || i < S) && member(key) && (key & pmask) == prefix)
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
    row.each([&](int i, unsigned key) { cnt += __popcll(__ballot((PADDED || i < S) && key == T)); });
    if (lane == 0) sm.wcnt[wave] = cnt;
    __syncthreads();
    int seen = 0;
    for (int w = 0; w < wave; w++) seen += sm.wcnt[w];
    row.each([&](int i, unsigned key) {
      const bool eq = (PADDED || i < S) && key == T;
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

// radix_threshold_of for the members of linear bin bstar.
template <int NT, int KREG, typename Load, typename SM>
__device__ __forceinline__ void radix_threshold(RowView<NT, KREG, Load>& row, int bstar, int rem,
                                                float lo, float scale, SM& sm,
                                                unsigned (*whist)[256]) {
  radix_threshold_of<NT, KREG>(
      row, [&](unsigned key) { return lin_bin(key_score(key), lo, scale) == bstar; }, rem, sm,
      whist);
}

// Steps 1 (after the histogram) to 3.  sm.hist holds the histogram of the
// row under (lo, scale) and sm.n_cand is 0; whist: the radix passes' per-wave
// histograms (NT/64 rows of 256 words of LDS; written only when the bin of
// the k-th score stays crowded).  All NT threads call it together.
template <int NT, int KREG, typename Load, typename SM>
__device__ __forceinline__ void select_from_histogram(RowView<NT, KREG, Load>& row, int k,
                                                      int32_t* out_idx, float* out_val,
                                                      SM& sm, float lo, float scale,
                                                      unsigned (*whist)[256]) {
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
    radix_threshold<NT, KREG>(row, bstar, rem0, lo, scale, sm, whist);
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

// The smallest key K in [a, b) (b <= 2^32) for which pred(K) holds, or b
// when none does; pred must be monotone on [a, b) (false, then true).  One
// wave searches 64-way: each round its lanes test 64 evenly spaced keys, so a
// 32-bit range takes six rounds.  Every lane returns the same value.
template <typename Pred>
__device__ __forceinline__ unsigned long long first_key_where(unsigned long long a,
                                                              unsigned long long b, Pred&& pred) {
  const unsigned long long lane = threadIdx.x & 63;
  unsigned long long lo = a, hi = b;  // the answer is in [lo, hi]; keys below lo fail
  while (lo < hi) {
    const unsigned long long n = hi - lo, step = (n + 63) >> 6;
    const unsigned long long cand = lo + lane * step;
    const unsigned long long m = __ballot(cand < hi && pred((unsigned)cand));
    if (m != 0ull) {
      const unsigned long long i0 = (unsigned long long)__builtin_ctzll(m);
      hi = lo + i0 * step;  // pred holds here
      if (i0 == 0) break;   // and at lo: lo is the answer
      lo += (i0 - 1) * step + 1;
    } else {
      const unsigned long long last = (n - 1) / step < 63 ? (n - 1) / step : 63;
      lo += last * step + 1;  // every tested key failed
    }
  }
  return hi;
}

// As first_key_where, but first testing the 64 keys around `guess` (the
// order key of the score at which pred is expected to turn true): when that
// window holds the turning point, one round decides; otherwise the search
// goes on above or below the window.
template <typename Pred>
__device__ __forceinline__ unsigned long long first_key_near(unsigned long long a,
                                                             unsigned long long b, unsigned guess,
                                                             Pred&& pred) {
  const unsigned long long lane = threadIdx.x & 63;
  unsigned long long w0 = guess >= 31u ? (unsigned long long)guess - 31 : 0ull;
  if (w0 < a) w0 = a;
  if (w0 >= b) return first_key_where(a, b, pred);
  const unsigned long long key = w0 + lane;
  const unsigned long long m = __ballot(key < b && pred((unsigned)key));
  if (m == 0ull) return first_key_where(w0 + 64 < b ? w0 + 64 : b, b, pred);  // all below
  if ((m & 1ull) == 0ull || w0 == a) return w0 + (unsigned long long)__builtin_ctzll(m);
  return first_key_where(a, w0, pred);  // pred holds at w0: the turning point is below
}

// The smallest key in [a, b) whose linear bin under (lo, scale) is at least
// target (b when none is): bins are monotone in the key.
__device__ __forceinline__ unsigned long long first_key_of_bin(unsigned long long a,
                                                               unsigned long long b, int target,
                                                               float lo, float scale) {
  if (target <= 0) return a;
  if (target >= kBins || scale == 0.f) return b;
  // the bin's lower edge in score space, a guess within a few ulps
  const unsigned guess = order_key(lo + (float)target / scale);
  return first_key_near(a, b, guess, [&](unsigned key) {
    return lin_bin(key_score(key), lo, scale) >= target;
  });
}

// Steps 1 (after the histogram) to 3 for a caller that needs the selected
// elements but not in index order (the attention over them).  The binning is
// monotone in the order key, so the members of the bin b* holding the k-th
// score are the keys of one interval [K_lo, K_hi] and the members of higher
// bins are the keys above K_hi: after the scan two waves find both ends
// (first_key_of_bin: one 64-key round near the bin's edge), and every pass
// over the keys compares integers.
//  * a crowded b* (more than kFewCandidates members) is split into kBins
//    linear sub-bins (one pass over the interval's keys and a scan) and the
//    interval narrowed to the sub-bin holding the k-th score; radix passes
//    over the interval's keys resolve a group still crowded after that;
//  * one pass counts, per wave, the keys above the interval (a ballot and a
//    scalar count per key slot) and copies the interval's keys, the
//    candidates, to LDS (rare: a slot holding some reserves consecutive
//    places at once); the candidates are ranked by (key descending, index
//    ascending) and the rem first are taken; (T, I) is the last taken;
//  * one pass writes the taken elements: element i with key > T, or
//    key == T and i <= I.  Key slot j of a wave holds 64 consecutive
//    indices, so one ballot per slot places them after the counts of the
//    waves and ballots before: the output is in ascending index order.
// The passes are bound by vector instructions per key (a wave64 instruction
// takes its SIMD four cycles), hence the scalar counts.
// Padding elements (index >= S) must have key 0 (RowView's load_score gives
// them the all-ones NaN, KeyRow key 0) and no score may have those bits: key
// 0 is then never taken and no pass checks the index.  sm.hist holds the
// histogram under (lo, scale) and sm.n_cand is 0; whist: the radix passes'
// per-wave histograms.  Writes k entries of out_idx / out_key (the taken
// indices, in ascending order, and their order keys) and sm.thr_key /
// sm.thr_idx = (T, I).  All NT threads; the caller needs a barrier before
// reading the output.
// mark(i) is called at three points (profiling builds record a time stamp):
// 0 the threshold group's keys known, 1 the last taken element known, 2 this
// wave's taken elements written.
template <int NT, int KREG, typename Row, typename SM, typename Mark>
__device__ __forceinline__ void select_keys(Row& row, int k, int32_t* out_idx, unsigned* out_key,
                                            SM& sm, float lo, float scale,
                                            unsigned (*whist)[256], Mark&& mark) {
  constexpr int NW = NT / 64;
  static_assert(NW >= 2, "two waves search the interval's ends");
  static_assert(KREG > 0 && KREG <= 32, "keys in registers, a bit per key of a thread");
  // the wave index in a scalar register: offsets and counts below stay scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  select_scan<NT>(sm, k);  // ends with a barrier
  const int bstar = sm.sel_bin;
  const int rem0 = k - sm.sel_gt;  // 1 <= rem0 <= members of b*
  int rem = rem0, nb = sm.sel_eq;
  // ---- the keys of b*: [K_lo, K_hi); K_hi = 2^32 when b* is the top bin
  if (wave < 2) {
    const unsigned long long e = first_key_of_bin(0ull, 1ull << 32, bstar + wave, lo, scale);
    if (lane == 0) {
      if (wave == 0)
        sm.key_lo = (unsigned)e;
      else
        sm.key_hi1 = (unsigned)(e - 1);  // K_hi >= 1: key 0 lies in bin 0
    }
  }
  __syncthreads();
  // key 0 belongs to the padding only
  unsigned klo = max(sm.key_lo, 1u), khi1 = sm.key_hi1;

  // ---- a crowded b*: linear sub-bins of its interval
  if (nb > kFewCandidates && scale > 0.f && scale * (float)kBins < INFINITY) {
    const float lo2 = lo + (float)bstar / scale, scale2 = scale * (float)kBins;
    for (int e = (int)threadIdx.x; e < kBins; e += NT) sm.hist[e] = 0u;
    __syncthreads();  // every thread has read the first scan's results
#pragma unroll
    for (int j = 0; j < KREG; j++) {
      const unsigned key = row.kv[j];
      if (key >= klo && key <= khi1) atomicAdd(&sm.hist[lin_bin(key_score(key), lo2, scale2)], 1u);
    }
    __syncthreads();
    select_scan<NT>(sm, rem0);
    const int sub = sm.sel_bin;
    rem = rem0 - sm.sel_gt;
    nb = sm.sel_eq;
    const unsigned long long a = klo, b = (unsigned long long)khi1 + 1;
    if (wave < 2) {
      const unsigned long long e = first_key_of_bin(a, b, sub + wave, lo2, scale2);
      if (lane == 0) {
        if (wave == 0)
          sm.key_lo = (unsigned)e;
        else
          sm.key_hi1 = (unsigned)(e - 1);  // e > a: the sub-bin has members
      }
    }
    __syncthreads();
    klo = max(sm.key_lo, 1u);
    khi1 = sm.key_hi1;
  }

  mark(0);
  // ---- the last taken element (T, I) and each wave's number of taken ones
  if (nb <= kFewCandidates) {
    const unsigned span = khi1 - klo;  // key - klo <= span: klo <= key <= khi1
    int gt = 0;                        // this wave's keys above the interval
#pragma unroll
    for (int j = 0; j < KREG; j++) {
      const unsigned key = row.kv[j];
      gt += __popcll(__ballot(key > khi1));
      const bool c = key - klo <= span;
      const unsigned long long m = __ballot(c);
      if (m != 0ull) {
        // rare: the slot's candidates take consecutive places (at most
        // kFewCandidates in all: the group's members are exactly the nb
        // elements its bin counted)
        int slot = 0;
        if (lane == 0) slot = atomicAdd(&sm.n_cand, __popcll(m));
        slot = __builtin_amdgcn_readfirstlane(slot);
        if (c) {
          const int at = slot + lane_rank(m);
          sm.cand_key[at] = key;
          sm.cand_idx[at] = row.base + j * 64;
        }
      }
    }
    if (lane == 0) sm.wcnt[wave] = gt;
    __syncthreads();
    // rank of candidate c = members ordered before it by (key descending,
    // index ascending): one ballot over the candidates on the lanes; the
    // waves take the candidates in turn; a taken one counts for its wave
    // (element i sits in wave i / per_wave)
    {
      const bool have = lane < nb;
      const unsigned mk = have ? sm.cand_key[lane] : 0u;
      const int mi = have ? sm.cand_idx[lane] : INT_MAX;
      for (int c = wave; c < nb; c += NW) {
        const unsigned ck = (unsigned)__builtin_amdgcn_readlane((int)mk, c);
        const int ci = __builtin_amdgcn_readlane(mi, c);
        const int rank = __popcll(__ballot(have && (mk > ck || (mk == ck && mi < ci))));
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
    radix_threshold_of<NT, KREG, true>(
        row, [&](unsigned key) { return key >= klo && key <= khi1; }, rem, sm, whist);
    const unsigned T = sm.thr_key;
    const int I = sm.thr_idx;
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KREG; j++) {
      const unsigned key = row.kv[j];
      cnt += __popcll(__ballot(key > T || (key == T && row.base + j * 64 <= I)));
    }
    if (lane == 0) sm.wcnt[wave] = cnt;
    __syncthreads();
  }

  mark(1);
  // ---- write the taken elements: key slot j of a wave holds 64 consecutive
  // indices, so a ballot per slot writes them in ascending index order
  const unsigned T = sm.thr_key;
  const int I = sm.thr_idx;
  int out = 0;
  for (int w = 0; w < wave; w++) out += sm.wcnt[w];
  const int ib = I - wave * row.per_wave;  // element i <= I: lane <= ib - 64 j
#pragma unroll
  for (int j = 0; j < KREG; j++) {
    const unsigned key = row.kv[j];
    // the ballot from the three comparisons' lane masks (scalar and / or),
    // the branch from the same comparisons
    const bool gt = key > T, eq = key == T, le = lane <= ib - j * 64;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(gt) |
                                 (__builtin_amdgcn_ballot_w64(eq) & __builtin_amdgcn_ballot_w64(le));
    if (gt || (eq && le)) {
      const int at = out + lane_rank(m);
      out_idx[at] = row.base + j * 64;
      out_key[at] = key;
    }
    out += __popcll(m);
  }
  mark(2);
}

template <int NT, int KREG, typename Row, typename SM>
__device__ __forceinline__ void select_keys(Row& row, int k, int32_t* out_idx, unsigned* out_key,
                                            SM& sm, float lo, float scale,
                                            unsigned (*whist)[256]) {
  select_keys<NT, KREG>(row, k, out_idx, out_key, sm, lo, scale, whist, [](int) {});
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
  select_from_histogram<NT, KREG>(row, k, out_idx, out_val, sm, lo, scale, sm.whist);
}

}  // namespace loki
