// The whole Loki decode step of one query head in one workgroup, for rows of
// up to 32768 cached tokens.
//
// Loki (poster page, "Visual Insights", Figure 1 right; "TL;DR"; briefgpt.xyz
// abstract): rotate the query into the PCA basis, score every cached token
// with the leading d coordinates, keep the top k, run exact attention with the
// full-dimensional keys of those k tokens.
//
// One launch and no intermediate buffer in HBM, as in the one-launch kernel
// of short rows (fused.hip), but one query head per workgroup and the whole
// row of scores in LDS (up to 128 KB of the 160 KB of a compute unit):
//  0. the query is rotated by P[kv] (all D coordinates, and the new key's
//     row when appending) while the first two panel batches are in flight;
//  1. the leading-dp panel of the (b, kv) keys is streamed with 16-byte loads,
//     two batches in flight, each score written to LDS; the first batch's
//     scores fix a binning range (for rows above 16384 tokens their mean +- 6
//     standard deviations within their min / max, so that a few heavy-hitter
//     scores do not crowd the bulk into few bins) and every later score is
//     added to the selection histogram as it is produced;
//  2. the scores become order keys in registers, the LDS that held them is
//     reused, and select_keys (select_core.h) writes the selected tokens, in
//     ascending order, and their low-dim partial logits (the index set, when
//     asked for, is a copy of that list);
//  3. block_attend (attend_core.h) gathers the selected key tails and value
//     rows: with the nontemporal policy for a single query head per KV head,
//     with the default one for grouped heads, whose siblings on the same XCD
//     select some of the same rows.
// Grouped query heads: the g heads of one (b, kv) are g workgroups on one XCD
// (workgroup i runs on XCD i % 8), each streaming the same panel with the
// default cache policy, so that the panel comes from HBM once and from that
// XCD's L2 for the other heads.  Few heads (fewer than the resident
// workgroup slots, single query head per KV head): spare slots run helpers,
// each repeating the rotation, scores and selection of one head (its panel
// from L2) and attending the second half of its rows; the later of the two
// merges the halves (the one-launch kernel's pairing, same flags and tags).
// Appending (poster page, "Loki's Computational Cost"): every workgroup of
// the (b, kv) rotates the new key as one more row, stores the same bytes at
// row S-1 of both caches and scores the new token from the rounded row; no
// wave reads row S-1 of the panel.
#include <type_traits>

#include "attend_core.h"
#include "loki_internal.h"
#include "phase_stamps.h"
#include "select_core.h"

namespace loki {

namespace {

constexpr int kHeadBatch = 8;         // 16-byte panel loads per lane per batch
constexpr int kHeadRowsPerBatch = 4;  // gather rows per lane group per batch
constexpr int kXcds = 8;              // MI355X: workgroup i runs on XCD i % 8
constexpr int kClampRows = 16384;     // rows above this bin over mean +- 6 sd

constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Byte offsets inside the reused LDS region, once the scores are in registers:
// selected tokens [k] i32, their partial logits [k] f32, the radix passes'
// per-wave histograms, the attention's merge.  Before that the region holds
// the row of scores, and before those the rotation's per-wave partial sums.
template <int DT, int D, int NT, int GR>
struct HeadLds {
  static constexpr int NW = NT / 64;
  __host__ __device__ static size_t slow(int k) { return align16((size_t)4 * k); }
  __host__ __device__ static size_t whist(int k) { return slow(k) + align16((size_t)4 * k); }
  __host__ __device__ static size_t att(int k) { return whist(k) + (size_t)NW * 256 * 4; }
  __host__ __device__ static size_t end(int k) { return att(k) + sizeof(AttendSmem<DT, D, NT>); }
  __host__ __device__ static size_t bytes(int S, int k) {
    const size_t sc = align16((size_t)4 * S), e = end(k), q = (size_t)NW * GR * D * 4;
    return sc > e ? (sc > q ? sc : q) : (e > q ? e : q);
  }
};

// Polls a flag until it holds tag, for at most `ticks` of the constant
// 100 MHz clock; true when it did.
__device__ __forceinline__ bool wait_flag(const unsigned long long* f, unsigned long long tag,
                                          unsigned long long ticks) {
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) return false;
    __builtin_amdgcn_s_sleep(4);
  }
  return true;
}

// A member of a pair sharing the stream is through with the hand-over (its
// half published, the other half read or scored itself).  xf[0], xf[1]: the
// members' flags; xf[2]: the tag of the first member through.  The second
// clears all three, so that a replay of a captured launch, which reuses the
// tag, starts afresh.
__device__ __forceinline__ void pair_share_done(unsigned long long* xf, unsigned long long tag) {
  if (__hip_atomic_exchange(xf + 2, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag) {
    __hip_atomic_store(xf + 0, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(xf + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(xf + 2, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// phase stamps (profiling builds): 0 start, 1 rotation done, 2 scores in
// LDS, 3 selection done, 4 attention starts, 5 end; pairs sharing the stream:
// 6 wave 0 through its half of the stream, 7 every wave through it, 8 the
// half published, 9 the partner's flag seen (or the wait over), 10 the
// partner's half in LDS, 11 written only when the wait timed out; inside
// the selection (wave 0): 12 threshold group known, 13 last taken element
// known, 14 taken elements written
LOKI_STAMP_ARRAY(g_stamps_head);

template <int DT, int D, int LPT, int NT, int KREG, bool APPEND>
__global__ __launch_bounds__(NT, 4) void head_kernel(HeadParams p) {
  constexpr int GR = APPEND ? 2 : 1;  // rows rotated: the query, then the new key
  constexpr int NW = NT / 64;
  constexpr int E = Elem<DT>::kPerVec;
  constexpr int DP = LPT * 16 / Elem<DT>::kBytes;  // panel width (== d)
  constexpr int TPP = NT / LPT;                    // tokens per pass over the panel
  // 512 threads (a thread holds 8 rows of P during the rotation): batches of
  // 4 loads, so that nothing spills (a spill reload waits for every load in
  // flight)
  constexpr int NB = NT >= 1024 ? kHeadBatch : kHeadBatch / 2;
  // rotation: 32 column quads x NT/32 row slots (D/4 <= 32 quads in use)
  constexpr int RSR = NT / 32, NR = (D + RSR - 1) / RSR;
  constexpr int NXV = (GR * D + NT - 1) / NT;
  static_assert(D % 4 == 0 && D <= 128, "at most 32 column quads");
  using L = HeadLds<DT, D, NT, GR>;

  extern __shared__ __align__(16) unsigned char reuse[];
  __shared__ SelectSmemLite<NW> ssm;
  __shared__ float xq[GR][D];           // the query row (and the new key), fp32
  __shared__ float qs[D];               // rotated query row
  __shared__ float kn[APPEND ? D : 1];  // rotated new key as stored
  __shared__ float rng[4][NW];          // per-wave min, max, sum, sum of squares
  __shared__ int later;                 // paired head: this workgroup merges the halves
  __shared__ int xok;                   // shared stream: the partner's half has arrived

  const Shape& sh = p.sh;
  const int S = sh.S, k = p.k;
  const int Ss = APPEND ? S - 1 : S;  // tokens read from the panel
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // [S] the scores as order keys (phase 1; -0 as +0): the selection loads
  // them as they are
  unsigned* sk = reinterpret_cast<unsigned*>(reuse);

  // ---- the query head of this workgroup
  int bh;  // b * Hq + h
  bool helper = false;
  if (sh.g == 1) {
    helper = (int)blockIdx.x >= p.n_heads;
    bh = helper ? p.help_first + ((int)blockIdx.x - p.n_heads) : (int)blockIdx.x;
  } else {
    // the g heads of (b, kv) unit u: workgroups (blk*g + j)*8 + u % 8, blk = u / 8
    const int x = (int)blockIdx.x % kXcds, s = (int)blockIdx.x / kXcds;
    const int u = (s / sh.g) * kXcds + x;
    if (u >= sh.B * sh.Hkv) return;  // padding of the last block of units
    bh = (u / sh.Hkv) * sh.Hq + (u % sh.Hkv) * sh.g + s % sh.g;
  }
  const int pair = bh - p.help_first;
  const bool paired = sh.g == 1 && p.n_help > 0 && pair >= 0 && pair < p.n_help;
  const int b = bh / sh.Hq, kv = (bh % sh.Hq) / sh.g;
  const size_t head = (size_t)b * sh.Hkv + kv;  // (b, kv) block of the caches
  // A head and its helper share out the stream (p.share): each streams one
  // half of the passes and hands its scores to the other through the
  // workspace.  Otherwise each streams the whole panel.
  const bool share = paired && p.share;
  const int member = helper ? 1 : 0;
  const int n_pass_all = (Ss + TPP - 1) / TPP;
  const int half = n_pass_all / 2;  // member 0: passes [0, half), member 1: the rest
  const int pass_lo = share && member ? half : 0;
  const int n_pass = share ? (member ? n_pass_all - half : half) : n_pass_all;
  const int t_lo = pass_lo * TPP, t_hi = min((pass_lo + n_pass) * TPP, Ss);
  // the panel is read again by a partner or by sibling heads: keep it in L2
  const bool keep_panel = (paired && !share) || sh.g > 1;

  // Phases 0 and 1 are built three times (the panel kept in L2; streamed
  // with the nontemporal policy; streamed and shared) and a workgroup takes
  // one: with the policy or the hand-over's stores chosen per load, the
  // compiler could not tell how many loads were in flight and waited for all
  // of them at every use (the rotation behind both first batches, every
  // batch behind the next one).
  float blo = 0.f, bscale = 0.f;  // binning range of the selection histogram
  float* const xrow = share ? p.xbuf + (size_t)bh * S : nullptr;  // scores handed over
  LOKI_STAMP(g_stamps_head, 0);
  LOKI_STAMP_HWID(g_stamps_head);
  auto phase01 = [&](auto keep_tag, auto share_tag) {
  constexpr bool KEEP = decltype(keep_tag)::value;
  constexpr bool SHARE = decltype(share_tag)::value;
  __builtin_amdgcn_s_setprio(3);
  // ---- 0. rotation: qs = q . P[kv] (and the new key's row), every column;
  // thread = (column quad cq, row slot rs), rows rs + RSR*u of P
  const Rsrc Prs = make_rsrc(p.P + (size_t)kv * D * D, (uint32_t)(D * D * 4));
  const int cq = tid % 32, rs = tid / 32;
  u32x4 pl[NR];
#pragma unroll
  for (int u = 0; u < NR; u++) {
    const int row = rs + RSR * u;
    pl[u] = load16(Prs, (row < D && 4 * cq < D) ? (row * D + 4 * cq) * 4 : kOutOfRange);
  }
  float xv[NXV];
#pragma unroll
  for (int u = 0; u < NXV; u++) {
    const int e = min(tid + u * NT, GR * D - 1);  // clamped: the load needs no branch
    if constexpr (APPEND)
      xv[u] = e < D ? load_elem<DT>(p.q, (size_t)bh * D + e)
                    : load_elem<DT>(p.k_new, head * D + (e - D));
    else
      xv[u] = load_elem<DT>(p.q, (size_t)bh * D + e);
  }
  using Raw = typename std::conditional<Elem<DT>::kBytes == 4, unsigned, unsigned short>::type;
  Raw vraw = 0;
  if constexpr (APPEND) vraw = static_cast<const Raw*>(p.v_new)[head * D + min(tid, D - 1)];
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the panel loads

  // ---- 1a. two panel batches in flight during the rotation
  const int c = tid % LPT, tl = tid / LPT;
  const Rsrc prs = make_rsrc(static_cast<const char*>(p.kcache) +
                                 head * sh.kl.head_elems * (size_t)Elem<DT>::kBytes,
                             (uint32_t)((size_t)sh.S_cap * LPT * 16));
  auto issue = [&](u32x4 (&x)[NB], int pass0) {
#pragma unroll
    for (int it = 0; it < NB; it++) {
      const int t = (pass_lo + pass0 + it) * TPP + tl;
      const uint32_t off = t < t_hi ? ((uint32_t)t * LPT + c) * 16 : kOutOfRange;
      x[it] = KEEP ? load16(prs, off) : load16_stream(prs, off);
    }
  };
  u32x4 xa[NB], xb[NB];
  // both batches in flight during the rotation while the P rows and the
  // batches fit 80 registers (1024 threads: 4 rows of P and two batches of 8
  // loads; 512 threads: 8 rows and two batches of 4)
  constexpr bool kEarlyB = NR * 4 + 2 * NB * 4 <= 80;
  issue(xa, 0);
  if constexpr (kEarlyB) issue(xb, NB);

#pragma unroll
  for (int u = 0; u < NXV; u++) {
    const int e = tid + u * NT;
    if (e < GR * D) xq[e / D][e % D] = xv[u];
  }
  select_clear<NT>(ssm);  // the histogram fills while scoring
  __syncthreads();
  {
    // per-wave partial rotations in the reused region (no score is there yet)
    auto qp = reinterpret_cast<float (*)[GR][D]>(reuse);
    float a[GR][4];
#pragma unroll
    for (int r = 0; r < GR; r++)
#pragma unroll
      for (int cc = 0; cc < 4; cc++) a[r][cc] = 0.f;
#pragma unroll
    for (int u = 0; u < NR; u++) {
      const int row = rs + RSR * u;
      float f[4];
      unpack16<F32>(pl[u], f);
#pragma unroll
      for (int r = 0; r < GR; r++) {
        const float x = row < D ? xq[r][row] : 0.f;
#pragma unroll
        for (int cc = 0; cc < 4; cc++) a[r][cc] = fmaf(x, f[cc], a[r][cc]);
      }
    }
    // the two row slots of a column quad in one wave are lanes cq and cq + 32
#pragma unroll
    for (int r = 0; r < GR; r++)
#pragma unroll
      for (int cc = 0; cc < 4; cc++) a[r][cc] += __shfl_xor(a[r][cc], 32, 64);
    if (lane < 32 && 4 * cq < D)
#pragma unroll
      for (int r = 0; r < GR; r++)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) qp[wave][r][4 * cq + cc] = a[r][cc];
    __syncthreads();
    for (int e = tid; e < GR * D; e += NT) {
      const int r = e / D, j = e % D;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; w++) s += qp[w][r][j];
      if (r == 0) {
        qs[j] = s;
      } else if (j < DP) {  // the new key's panel coordinate: stored, and kept as stored
        store_elem<DT>(p.kcache, head * sh.kl.head_elems + (size_t)(S - 1) * DP + j, s);
        kn[j] = stored_value<DT>(s);
      } else {  // the rest of the new key's row
        store_elem<DT>(p.kcache, head * sh.kl.head_elems + sh.kl.rest_off +
                                     (size_t)(S - 1) * (D - DP) + (j - DP), s);
      }
    }
    if constexpr (APPEND)
      if (tid < D) static_cast<Raw*>(p.vcache)[(head * sh.S_cap + (size_t)(S - 1)) * D + tid] = vraw;
    __syncthreads();
  }
  if constexpr (!kEarlyB) issue(xb, NB);

  LOKI_STAMP(g_stamps_head, 1);
  __builtin_amdgcn_s_setprio(0);
  // ---- 1b. low-dim scores of every token into LDS, the histogram built as
  // they are produced (after the first batch has fixed the binning range)
  const bool clamp = S > kClampRows;
  float lo = INFINITY, hi = -INFINITY, sum = 0.f, sq = 0.f;
  {
    float qv[E];
#pragma unroll
    for (int e = 0; e < E; e++) qv[e] = qs[c * E + e];  // c*E < DP == d
    if constexpr (APPEND) {
      // score of the new token from its stored panel coordinates, summed as
      // the stream sums a row (lane partials, then pairwise sums)
      if (wave == 0) {
        const int cl = lane % LPT;
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) a = fmaf(qs[cl * E + e], kn[cl * E + e], a);
        a = group_sum<LPT>(a);
        if (lane == 0) {
          sk[S - 1] = order_key_nz(a + 0.f);
          lo = fminf(lo, a);
          hi = fmaxf(hi, a);
        }
      }
    }
    // a finished score r of token t (t_lo <= t < t_hi)
    auto put = [&](int t, float r, bool hist, bool first) {
      if (first) {
        lo = fminf(lo, r);
        hi = fmaxf(hi, r);
        sum += r;
        sq = fmaf(r, r, sq);
      }
      sk[t] = order_key_nz(r + 0.f);  // + 0 turns -0 into +0
      if (hist) atomicAdd(&ssm.hist[lin_bin(r, blo, bscale)], 1u);
    };
    auto consume = [&](const u32x4 (&x)[NB], int pass0, bool hist, bool first) {
      if constexpr (LPT == 4 && NB % 4 == 0) {
        // lane partials, then a reduce-scatter over groups of 4 passes: lane c
        // of a quad ends with the whole score of pass (group + c) (pairs added
        // as in group_sum<4>)
        float a[NB];
#pragma unroll
        for (int it = 0; it < NB; it++) {
          float f[E];
          unpack16<DT>(x[it], f);
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < E; e++) acc = fmaf(qv[e], f[e], acc);
          a[it] = acc;
        }
        const bool b0 = (c & 1) != 0, b1 = (c & 2) != 0;
#pragma unroll
        for (int g0 = 0; g0 < NB; g0 += 4) {
          const float u0 = (b0 ? a[g0 + 1] : a[g0]) + dpp_f<0xB1>(b0 ? a[g0] : a[g0 + 1]);
          const float u1 = (b0 ? a[g0 + 3] : a[g0 + 2]) + dpp_f<0xB1>(b0 ? a[g0 + 2] : a[g0 + 3]);
          const float r = (b1 ? u1 : u0) + dpp_f<0x4E>(b1 ? u0 : u1);
          const int t = (pass_lo + pass0 + g0 + c) * TPP + tl;
          if (t < t_hi) put(t, r, hist, first);
        }
      } else {
#pragma unroll
        for (int it = 0; it < NB; it++) {
          float f[E];
          unpack16<DT>(x[it], f);
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < E; e++) a = fmaf(qv[e], f[e], a);
          a = group_sum<LPT>(a);
          const int t = (pass_lo + pass0 + it) * TPP + tl;
          if (t < t_hi && c == 0) put(t, a, hist, first);
        }
      }
    };
    consume(xa, 0, false, true);
    {
      // the binning range from the first batch of scores (and the new token)
      const float l0 = -wave_max(-lo), h0 = wave_max(hi);
      const float s0 = wave_sum(sum), q0 = wave_sum(sq);
      if (lane == 0) {
        rng[0][wave] = l0;
        rng[1][wave] = h0;
        rng[2][wave] = s0;
        rng[3][wave] = q0;
      }
      __syncthreads();
      blo = rng[0][0];
      float bhi = rng[1][0], s1 = rng[2][0], s2 = rng[3][0];
#pragma unroll
      for (int w = 1; w < NW; w++) {
        blo = fminf(blo, rng[0][w]);
        bhi = fmaxf(bhi, rng[1][w]);
        s1 += rng[2][w];
        s2 += rng[3][w];
      }
      if (clamp) {
        // mean +- 6 sd of the first batch, within its min / max; scores
        // outside land in the end bins (clamped bins stay monotone); a
        // non-finite mean or spread leaves the range as it is
        const float n1 = (float)min(t_hi - t_lo, NB * TPP);
        const float mean = s1 / n1;
        const float sd = sqrtf(fmaxf(s2 / n1 - mean * mean, 0.f));
        blo = fmaxf(blo, mean - 6.f * sd);
        bhi = fminf(bhi, mean + 6.f * sd);
      }
      bscale = bin_scale(blo, bhi);
      for (int t = t_lo + tid; t < min(t_hi, t_lo + NB * TPP); t += NT)
        atomicAdd(&ssm.hist[lin_bin(key_score(sk[t]), blo, bscale)], 1u);
      if (APPEND && tid == 0)  // the new token (never streamed)
        atomicAdd(&ssm.hist[lin_bin(key_score(sk[S - 1]), blo, bscale)], 1u);
    }
    // every batch is issued, also past the end (those loads are out of range:
    // zeros, no memory access), so that the loads in flight are the same on
    // every path and each use waits only for its own batch
    // (the scheduling barriers keep each batch's use after the issue of the
    // next one: hoisted above it, the use would wait for every load)
    issue(xa, 2 * NB);
    __builtin_amdgcn_sched_barrier(0);
    consume(xb, NB, true, false);
    issue(xb, 3 * NB);
    __builtin_amdgcn_sched_barrier(0);
    for (int pass = 2 * NB; pass < n_pass; pass += 2 * NB) {
      consume(xa, pass, true, false);
      issue(xa, pass + 2 * NB);
      __builtin_amdgcn_sched_barrier(0);
      consume(xb, pass + NB, true, false);
      issue(xb, pass + 3 * NB);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SHARE) {
      // ---- 1c. the hand-over: this half of the row goes out through the
      // workspace (agent-coherent words), the other half comes in.  The
      // stores wait for the end of the stream: issued among its loads, or by
      // waves already through it, they slowed the stream down by more than
      // they saved (measured)
      LOKI_STAMP(g_stamps_head, 6);
      __syncthreads();  // this half's scores are in LDS
      LOKI_STAMP(g_stamps_head, 7);
      for (int t = t_lo + tid; t < t_hi; t += NT) st_coherent(xrow + t, __uint_as_float(sk[t]));
      wait_stores();
      __syncthreads();  // every store of this half is complete
      LOKI_STAMP(g_stamps_head, 8);
      unsigned long long* xf = p.xflag + (size_t)pair * 4;
      if (tid == 0) {
        __hip_atomic_store(xf + member, p.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        xok = wait_flag(xf + (1 - member), p.tag, p.wait_ticks);
      }
      __syncthreads();
      LOKI_STAMP(g_stamps_head, 9);
      if (!xok) LOKI_STAMP(g_stamps_head, 11);  // the partner's half is scored here
      const int u_lo = member ? 0 : half * TPP, u_hi = member ? half * TPP : Ss;
      if (xok) {
        // 16-byte agent-coherent loads (sc1), four in flight per thread, over
        // the 16-byte quads that hold the half (quads counted from the
        // 16-byte boundary at or below the row's start; words outside the
        // half are not used)
        const int sft = (int)(((size_t)bh * S) & 3);
        const Rsrc xr = make_rsrc(xrow - sft, (uint32_t)((S + sft) * 4));
        const int q_lo = (u_lo + sft) >> 2, q_hi = (u_hi + sft + 3) >> 2;
        for (int q0 = q_lo + tid; q0 < q_hi; q0 += 4 * NT) {
          u32x4 r[4];
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int qi = q0 + q * NT;
            r[q] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           xr, qi < q_hi ? (int)(16 * qi) : (int)kOutOfRange, 0, kCoherentSc1));
          }
#pragma unroll
          for (int q = 0; q < 4; q++) {
#pragma unroll
            for (int e = 0; e < 4; e++) {
              const int t = 4 * (q0 + q * NT) + e - sft;
              if (t >= u_lo && t < u_hi) {
                sk[t] = r[q][e];
                atomicAdd(&ssm.hist[lin_bin(key_score(r[q][e]), blo, bscale)], 1u);
              }
            }
          }
        }
      } else {
        // the partner has not published in time (not resident yet): its
        // half is scored here, with the same sums (group_sum adds the lanes'
        // partials as the stream's reduce-scatter does)
        for (int pass = u_lo / TPP; pass * TPP < u_hi; pass++) {
          const int t = pass * TPP + tl;
          const u32x4 x =
              load16_stream(prs, t < u_hi ? ((uint32_t)t * LPT + c) * 16 : kOutOfRange);
          float f[E];
          unpack16<DT>(x, f);
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < E; e++) a = fmaf(qv[e], f[e], a);
          a = group_sum<LPT>(a);
          if (c == 0 && t < u_hi) {
            sk[t] = order_key_nz(a + 0.f);
            atomicAdd(&ssm.hist[lin_bin(a, blo, bscale)], 1u);
          }
        }
      }
      LOKI_STAMP(g_stamps_head, 10);
      if (tid == 0) pair_share_done(xf, p.tag);
    }
  }
  };
  if (share)
    phase01(std::false_type{}, std::true_type{});
  else if (keep_panel)
    phase01(std::true_type{}, std::false_type{});
  else
    phase01(std::false_type{}, std::false_type{});

  __builtin_amdgcn_s_setprio(3);
  __syncthreads();  // every score is in LDS
  LOKI_STAMP(g_stamps_head, 2);

  // ---- 2. top-k: the order keys in registers, then the LDS reused
  int* sidx = reinterpret_cast<int*>(reuse);                         // [k]
  unsigned* skey = reinterpret_cast<unsigned*>(reuse + L::slow(k));  // [k] their keys
  auto whist = reinterpret_cast<unsigned (*)[256]>(reuse + L::whist(k));
  auto& asm_ = *reinterpret_cast<AttendSmem<DT, D, NT>*>(reuse + L::att(k));
  {
    KeyRow<NT, KREG> row(sk, S);  // elements past the row: key 0 (select_keys)
    __syncthreads();              // every key is in registers: the row's LDS is free
    select_keys<NT, KREG>(row, k, sidx, skey, ssm, blo, bscale, whist,
                          [&](int i) { LOKI_STAMP(g_stamps_head, 12 + i); });
  }
  LOKI_STAMP(g_stamps_head, 3);
  if constexpr (APPEND) {
    // the gathers may read row S-1: this wave's stores of it are complete
    // before the barrier that follows
    wait_stores();
  }
  __syncthreads();
  // the index set, when asked for: the selected list is in ascending order
  if (p.idx_out && !helper)
    for (int e = tid; e < k; e += NT) p.idx_out[(size_t)bh * k + e] = sidx[e];

  LOKI_STAMP(g_stamps_head, 4);
  __builtin_amdgcn_s_setprio(0);
  // ---- 3. exact attention over the selected tokens
  const int r0 = paired && helper ? p.k0 : 0;
  const int nr = paired ? (helper ? k - p.k0 : p.k0) : k;
  float M, Lsum, A;
  if (sh.g > 1)  // grouped heads: rows selected by several heads of a group come from L2
    block_attend<DT, D, NT, true, kHeadRowsPerBatch, false, false>(
        qs, p.scale_log2, sidx + r0, skey + r0, nr, p.kcache, p.vcache, head, sh, asm_, M, Lsum,
        A);
  else
    block_attend<DT, D, NT, true, kHeadRowsPerBatch, false, true>(
        qs, p.scale_log2, sidx + r0, skey + r0, nr, p.kcache, p.vcache, head, sh, asm_, M, Lsum,
        A);
  if (paired) {
    // owner: rows [0, k0); helper: rows [k0, k).  Partials (M, L, A[D]) of
    // pair j: owner's at help_part[2j], helper's at help_part[2j+1].
    float* mine = p.help_part + ((size_t)pair * 2 + (helper ? 1 : 0)) * (D + 2);
    const float* other = p.help_part + ((size_t)pair * 2 + (helper ? 0 : 1)) * (D + 2);
    if (tid < D) st_coherent(mine + 2 + tid, A);
    if (tid == 0) {
      st_coherent(mine, M);
      st_coherent(mine + 1, Lsum);
    }
    wait_stores();
    __syncthreads();
    if (tid == 0) {
      later = __hip_atomic_exchange(p.help_flag + pair, p.tag, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == p.tag;
      // both halves are in: the flag goes back to 0 (a replay of a captured
      // launch reuses its tag)
      if (later)
        __hip_atomic_store(p.help_flag + pair, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (later && tid < D) {
      const float oM = ld_coherent(other), oL = ld_coherent(other + 1);
      const float oA = ld_coherent(other + 2 + tid);
      // always the owner's half first: the result does not depend on which merges
      store_out(p.out, (size_t)bh * D + tid,
                helper ? combine_partials(oM, oL, oA, M, Lsum, A)
                       : combine_partials(M, Lsum, A, oM, oL, oA),
                sh.odt);
    }
  } else if (tid < D) {
    store_out(p.out, (size_t)bh * D + tid, A / Lsum, sh.odt);
  }
  LOKI_STAMP(g_stamps_head, 5);
}

// Threads per workgroup for rows of S tokens: 512 (two workgroups per
// compute unit) while a row's scores fit half of the LDS, else 1024.
int head_threads(int S) { return S <= 512 * 32 && S * 4 <= 64 * 1024 ? 512 : 1024; }

template <int DT, int D, int LPT, int NT, int KREG, bool APPEND>
hipError_t launch_v(const HeadParams& p, hipStream_t st) {
  const size_t dyn = HeadLds<DT, D, NT, APPEND ? 2 : 1>::bytes(p.sh.S, p.k);
  const dim3 grid((unsigned)(p.n_slots + p.n_help));
  head_kernel<DT, D, LPT, NT, KREG, APPEND><<<grid, NT, dyn, st>>>(p);
  return hipGetLastError();
}

// Order keys per thread in the selection: the fewest that hold the row, so
// that every wave of a short row holds keys (a wave owns KREG * 64
// consecutive tokens).
template <int DT, int D, int LPT, bool APPEND>
hipError_t launch_a(const HeadParams& p, hipStream_t st) {
  const int S = p.sh.S;
  if (head_threads(S) == 1024) return launch_v<DT, D, LPT, 1024, 32, APPEND>(p, st);
  if (S <= 512 * 8) return launch_v<DT, D, LPT, 512, 8, APPEND>(p, st);
  if (S <= 512 * 16) return launch_v<DT, D, LPT, 512, 16, APPEND>(p, st);
  return launch_v<DT, D, LPT, 512, 32, APPEND>(p, st);
}

template <int DT, int D, int LPT>
hipError_t launch_lpt(const HeadParams& p, hipStream_t st) {
  return p.k_new ? launch_a<DT, D, LPT, true>(p, st) : launch_a<DT, D, LPT, false>(p, st);
}

template <int DT, int D>
hipError_t launch_d(const HeadParams& p, hipStream_t st) {
  const int lpt = p.sh.dp * Elem<DT>::kBytes / 16;
  return lpt == 4 ? launch_lpt<DT, D, 4>(p, st) : launch_lpt<DT, D, 8>(p, st);
}

template <int DT>
hipError_t launch_dt(const HeadParams& p, hipStream_t st) {
  return p.sh.D == 96 ? launch_d<DT, 96>(p, st) : launch_d<DT, 128>(p, st);
}

// Static LDS of a built variant (the compiler's figure), read once.
template <int DT, int D, int LPT, int NT, bool APPEND>
size_t static_lds() {
  static const size_t bytes = [] {
    hipFuncAttributes a{};
    if (hipFuncGetAttributes(&a, reinterpret_cast<const void*>(
                                     &head_kernel<DT, D, LPT, NT, 32, APPEND>)) != hipSuccess)
      return (size_t)1 << 30;  // unknown: the variant is not used
    return (size_t)a.sharedSizeBytes;
  }();
  return bytes;
}

// LDS of the appending variant (the larger one) that a shape would take:
// dynamic + static bytes.
template <int DT, int D, int LPT>
size_t lds_for(const Shape& sh, int k) {
  if (head_threads(sh.S) == 512)
    return HeadLds<DT, D, 512, 2>::bytes(sh.S, k) + static_lds<DT, D, LPT, 512, true>();
  return HeadLds<DT, D, 1024, 2>::bytes(sh.S, k) + static_lds<DT, D, LPT, 1024, true>();
}

template <int DT>
size_t lds_dt(const Shape& sh, int k) {
  const int lpt = sh.dp * Elem<DT>::kBytes / 16;
  if (sh.D == 96) return lpt == 4 ? lds_for<DT, 96, 4>(sh, k) : lds_for<DT, 96, 8>(sh, k);
  return lpt == 4 ? lds_for<DT, 128, 4>(sh, k) : lds_for<DT, 128, 8>(sh, k);
}

}  // namespace

int head_kernel_threads(const Shape& sh) { return head_threads(sh.S); }

bool head_share_ok(const Shape& sh, int streamed) {
  const int nt = head_threads(sh.S);
  const int lpt = sh.dp * (sh.dtype == F32 ? 4 : 2) / 16;
  const int nb = nt >= 1024 ? kHeadBatch : kHeadBatch / 2;
  const int passes = (streamed + nt / lpt - 1) / (nt / lpt);
  return passes >= 4 * nb;
}

bool head_supported(const Shape& sh, int d, int k) {
  const int eb = sh.dtype == F32 ? 4 : 2;
  const int lpt = sh.dp * eb / 16;
  if (!(d == sh.dp && (sh.D == 128 || sh.D == 96) && (lpt == 4 || lpt == 8) &&
        sh.S <= 1024 * 32 && k >= 1))
    return false;
  // the appending variant (the larger) must fit the compute unit's LDS
  size_t lds = 0;
  switch (sh.dtype) {
    case F32: lds = lds_dt<F32>(sh, k); break;
    case F16: lds = lds_dt<F16>(sh, k); break;
    default: lds = lds_dt<BF16>(sh, k); break;
  }
  return lds <= 160 * 1024;
}

hipError_t launch_head(const HeadParams& p, hipStream_t st) {
  switch (p.sh.dtype) {
    case F32: return launch_dt<F32>(p, st);
    case F16: return launch_dt<F16>(p, st);
    default: return launch_dt<BF16>(p, st);
  }
}

}  // namespace loki

LOKI_STAMP_EXPORT(loki_phase_stamps_head, loki::g_stamps_head);
