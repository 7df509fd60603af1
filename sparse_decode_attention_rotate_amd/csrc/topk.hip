// Per-(batch, query head) top-k selection by approximate score.
//
// Loki (briefgpt.xyz abstract; poster page "TL;DR" and Figure 1 right): the
// tokens of the KV-cache are ranked by their low-dimensional scores and only
// the top k are kept for the exact attention.
//
// Exact radix select in one workgroup per row of scores:
//  * each fp32 score maps to an order-preserving 32-bit key (-0 folded to +0);
//  * up to four passes over 8-bit digits, most significant first, each
//    building per-wave LDS histograms of the keys that still share the
//    selected prefix; wave 0 finds the digit holding the k-th largest key with
//    a DPP prefix scan over the 256 bins (descending digit order);
//  * the pass loop stops early once every key sharing the prefix is selected;
//  * a final ordered compaction (wave ballots + mbcnt ranks) writes the
//    selected indices in ascending order: all keys above the threshold, and
//    the lowest-index keys equal to it (ties go to the lower index).
// Keys stay in registers across passes when S <= threads * KREG.
#include "loki_internal.h"

namespace loki {

namespace {

__device__ __forceinline__ unsigned order_key(float s) {
  unsigned u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// inverse of order_key (a -0 score comes back as +0)
__device__ __forceinline__ float key_value(unsigned key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

template <int NT, int KREG>
__global__ __launch_bounds__(NT) void topk_kernel(TopkParams p) {
  constexpr int NW = NT / 64;
  __shared__ unsigned hist[NW][256];
  __shared__ unsigned sel_digit, sel_gt, sel_eq;
  __shared__ int wcnt[2][NW][2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = p.S;
  const float* srow = p.scores + (size_t)blockIdx.x * S;

  // all score loads of this thread in flight at once (out-of-range ones read 0)
  const Rsrc srs = make_rsrc(srow, (uint32_t)S * 4u);
  unsigned keys[KREG > 0 ? KREG : 1];
  if constexpr (KREG > 0) {
    float sv[KREG];
#pragma unroll
    for (int j = 0; j < KREG; j++) {
      const int i = tid + j * NT;
      sv[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          srs, i < S ? (int)(i * 4) : (int)kOutOfRange, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < KREG; j++) keys[j] = order_key(sv[j]);
  }
  auto key_of = [&](int j, int i) -> unsigned {
    if constexpr (KREG > 0)
      return keys[j];
    else
      return order_key(srow[i]);
  };
  const int nj = (S + NT - 1) / NT;

  unsigned prefix = 0u, pmask = 0u;
  int rem = p.k;
  for (int pass = 0; pass < 4; pass++) {
    const int shift = 24 - 8 * pass;
    for (int e = tid; e < NW * 256; e += NT) (&hist[0][0])[e] = 0u;
    __syncthreads();
    if constexpr (KREG > 0) {
#pragma unroll
      for (int j = 0; j < KREG; j++) {
        const int i = tid + j * NT;
        if (i < S && (keys[j] & pmask) == prefix)
          atomicAdd(&hist[wave][(keys[j] >> shift) & 0xffu], 1u);
      }
    } else {
      for (int j = 0; j < nj; j++) {
        const int i = tid + j * NT;
        if (i < S) {
          const unsigned key = key_of(j, i);
          if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 0xffu], 1u);
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane holds digits 255-4*lane .. 252-4*lane (descending)
      unsigned c[4];
      unsigned tot = 0u;
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int dg = 255 - (lane * 4 + u);
        unsigned s = 0u;
#pragma unroll
        for (int w = 0; w < NW; w++) s += hist[w][dg];
        c[u] = s;
        tot += s;
      }
      unsigned before = wave_incl_scan(tot) - tot;  // keys with a larger digit
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const unsigned after = before + c[u];
        if (before < (unsigned)rem && after >= (unsigned)rem) {
          sel_digit = 255u - (unsigned)(lane * 4 + u);
          sel_gt = before;
          sel_eq = c[u];
        }
        before = after;
      }
    }
    __syncthreads();
    rem -= (int)sel_gt;
    prefix |= sel_digit << shift;
    pmask |= 0xffu << shift;
    const bool done = (int)sel_eq == rem;  // the whole equal-prefix group is taken
    __syncthreads();                         // sel_* and hist are rewritten next pass
    if (done) break;
  }

  // ordered compaction, ascending index
  int eq_seen = 0, out_seen = 0;
  int32_t* irow = p.idx + (size_t)blockIdx.x * p.k;
  float* vrow = p.sel_scores ? p.sel_scores + (size_t)blockIdx.x * p.k : nullptr;
  for (int j = 0; j < nj; j++) {
    const int i = tid + j * NT;
    const bool valid = i < S;
    unsigned key = 0u;
    if constexpr (KREG > 0) {
#pragma unroll
      for (int jj = 0; jj < KREG; jj++)
        if (jj == j) key = keys[jj];
    } else {
      key = valid ? key_of(j, i) : 0u;
    }
    const unsigned mk = key & pmask;
    const bool gt = valid && mk > prefix;
    const bool eq = valid && mk == prefix;
    const unsigned long long bg = __ballot(gt), be = __ballot(eq);
    const int buf = j & 1;
    if (lane == 0) {
      wcnt[buf][wave][0] = __popcll(bg);
      wcnt[buf][wave][1] = __popcll(be);
    }
    __syncthreads();
    int sel_before = 0, eq_before = 0, tot_eq = 0, tot_sel = 0;
    for (int w = 0; w < NW; w++) {
      const int cg = wcnt[buf][w][0], ce = wcnt[buf][w][1];
      int take = rem - (eq_seen + tot_eq);
      take = take < 0 ? 0 : (take > ce ? ce : take);
      if (w < wave) {
        sel_before += cg + take;
        eq_before += ce;
      }
      tot_eq += ce;
      tot_sel += cg + take;
    }
    const int eq_rank = eq_seen + eq_before + lane_rank(be);
    const bool sel = gt || (eq && eq_rank < rem);
    const unsigned long long bs = __ballot(sel);
    const int pos = out_seen + sel_before + lane_rank(bs);
    if (sel && pos < p.k) {  // exactly k are selected; the bound only guards the row
      irow[pos] = i;
      if (vrow) vrow[pos] = key_value(key);
    }
    eq_seen += tot_eq;
    out_seen += tot_sel;
  }
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, int n_rows, hipStream_t st) {
  const dim3 grid((unsigned)n_rows);
  if (p.S <= 512 * 16)
    topk_kernel<512, 16><<<grid, 512, 0, st>>>(p);
  else if (p.S <= 1024 * 32)
    topk_kernel<1024, 32><<<grid, 1024, 0, st>>>(p);
  else
    topk_kernel<1024, 0><<<grid, 1024, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace loki
