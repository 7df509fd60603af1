// The whole Loki decode step for one (batch, KV head) in one workgroup.
//
// Loki (poster page, "Visual Insights", Figure 1 right; "TL;DR"; briefgpt.xyz
// abstract): rotate the query into the PCA basis, score every cached token
// with the leading d coordinates, keep the top k, run exact attention with the
// full-dimensional keys of those k tokens.
//
// One launch, no intermediate buffers in HBM: per unit (b, kv) with its g
// query heads,
//  0. the panel coordinates of the query rows are rotated by P[kv] (16-byte
//     loads of P's leading dp columns, partial sums reduced across lanes and
//     waves) while the first two panel batches are already in flight;
//  1. the contiguous leading-dp panel of the unit's keys is streamed with
//     16-byte loads, two batches in flight, the g score rows kept in LDS and
//     their min / max folded on the way;
//  0'. the loads for the remaining D-dp coordinates of the rotation are issued
//     and stay in flight through the top-k;
//  2. top-k from LDS: a single head's scores are stored as order keys while
//     streaming (its histogram built as they come) and select_keys
//     (select_core.h) takes them from registers; several heads' scores go
//     through block_select one head at a time;
//  3. block_attend (attend_core.h) gathers the selected key tails and value
//     rows and writes the output rows.
// A decode step becomes one kernel: no launch gaps, no ramp-up/drain between
// phases, and the scores never leave LDS.  Used when d == dp, the unit's g
// score rows fit the LDS budget and S <= 4096.
//
// The appending variant (poster page, "Loki's Computational Cost": the
// KV-cache append belongs to every step) also takes the step's new key and
// value as token S-1: the key is rotated as one more row of phases 0 and 0'
// (same P loads), rounded to the storage dtype and written to row S-1 of the
// cache, the value row is copied, and the panel stream stops at S-1.  The new
// token's score comes from the rounded key in LDS with the lane partials and
// pairwise sums of the panel stream, so it is the score a later step computes
// from the stored row; no wave reads row S-1 of the panel.  Every wave waits
// for its stores before the barrier ahead of the attention, whose gathers may
// read the new row.
#include <type_traits>

#include "attend_core.h"
#include "loki_internal.h"
#include "phase_stamps.h"
#include "select_core.h"

namespace loki {

namespace {

// 256 threads when the units fill the GPU several times over, 512 when there
// are no more units than compute units (more loads in flight per unit).
constexpr int kFusedMaxS = 4096;          // scores of a unit held in registers for select
constexpr int kFusedBatch = 8;            // 16-byte panel loads per lane per batch
constexpr size_t kFusedDynBytes = 36 * 1024;
constexpr int kFusedRowsPerBatch = 4;  // gather rows per lane group per batch

// phase stamps (profiling builds): 0 start, 1 rotation done, 2 wave 0's
// scores in LDS, 3 selection (and the rest of the rotation) done, 4 end,
// 5 every wave's scores in LDS; inside the single-head selection (wave 0):
// 6 threshold group known, 7 last taken element known, 8 taken elements
// written
LOKI_STAMP_ARRAY(g_stamps_fused);

template <int DT, int D, int LPT, int G, int NT, bool APPEND>
__global__ __launch_bounds__(NT, NT == 256 ? 3 : 2) void fused_kernel(FusedParams p) {
  constexpr int GR = G + (APPEND ? 1 : 0);  // rows rotated: the queries, then the new key
  constexpr int NW = NT / 64;
  constexpr int KREG = kFusedMaxS / NT;  // order keys per thread in the selection
  constexpr int E = Elem<DT>::kPerVec;
  constexpr int DP = LPT * 16 / Elem<DT>::kBytes;  // panel width (== d)
  constexpr int TPP = NT / LPT;                    // tokens per pass over the panel
  constexpr int NB = kFusedBatch;
  // rotation of the panel coordinates: thread = (column quad, row slot)
  constexpr int NQL = DP / 4, RSL = NT / NQL, NL = D / RSL;
  // rotation of the remaining coordinates: 32 quad slots x 8 row slots
  constexpr int NQR = (D - DP) / 4, RSR = NT / 32, NR = D / RSR;
  static_assert(NT % NQL == 0 && D % RSL == 0 && NQR <= 32 && D % RSR == 0, "rotation tiling");
  static_assert(G * LPT <= 64, "the new token's score is formed by one wave");

  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ SelectSmem<NW> ssm;
  __shared__ AttendSmem<DT, D, NT> asm_;
  __shared__ float xq[GR][D];            // query rows (and the new key), fp32
  __shared__ float qpart[NW][GR][D];     // per-wave partial rotations
  __shared__ float qs[G][D];             // rotated query rows
  __shared__ float kn[APPEND ? D : 1];   // rotated new key as stored
  __shared__ float rng[2][NW][G];        // per-wave score min / max
  __shared__ int later;                  // paired unit: this workgroup merges the halves

  const Shape& sh = p.sh;
  const int S = sh.S, k = p.k;
  const int Ss = APPEND ? S - 1 : S;  // tokens read from the panel
  float* sc = reinterpret_cast<float*>(dyn);             // [G][S]
  // single head: the scores as order keys (-0 as +0), which the selection
  // loads as they are
  unsigned* sk = reinterpret_cast<unsigned*>(dyn);
  int* sidx = reinterpret_cast<int*>(sc + G * S);        // [G][k]
  float* slow = reinterpret_cast<float*>(sidx + G * k);  // [G][k]

  LOKI_STAMP(g_stamps_fused, 0);
  LOKI_STAMP_HWID(g_stamps_fused);
  // Wave priority: the short latency-bound phases (rotation, top-k) run at
  // high priority so that they are not starved of issue slots by the
  // streaming phases of co-resident workgroups; streaming runs at the lowest.
  __builtin_amdgcn_s_setprio(3);

  // The unit of this workgroup.  Workgroups past the last unit are helpers:
  // helper j repeats the rotation, scores and top-k of unit help_first + j
  // (same code, same data, same rows) and attends the second half of its
  // selected rows while the unit's own workgroup attends the first half; the
  // later of the two merges the halves.  Only single-head units are paired.
  const bool helper = (int)blockIdx.x >= p.n_units;
  const size_t head = helper ? (size_t)(p.help_first + ((int)blockIdx.x - p.n_units))
                             : (size_t)blockIdx.x;  // b * Hkv + kv
  const int pair = (int)head - p.help_first;
  const bool paired = G == 1 && p.n_help > 0 && pair >= 0 && pair < p.n_help;
  const int b = (int)(head / sh.Hkv), kv = (int)(head % sh.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t q0 = (size_t)b * sh.Hq + (size_t)kv * G;  // first query head of the group

  const Rsrc Prs = make_rsrc(p.P + (size_t)kv * D * D, (uint32_t)(D * D * 4));
  // Phases 0 and 1 are built twice, once per panel cache policy, and a
  // workgroup takes one: with the policy chosen per load, the compiler could
  // not tell how many loads were in flight and waited for all of them at
  // every use (the rotation behind both first batches, every batch behind the
  // next one).
  float lo[G], hi[G];
  float blo = 0.f, bscale = 0.f;  // binning of the single-head histogram
  auto phase01 = [&](auto keep_tag) {
  constexpr bool KEEP = decltype(keep_tag)::value;
  // ---- 0. rotation of the panel coordinates: qs[h][0:DP] = q[h] . P[kv][:, 0:DP]
  // Its loads go out first: a wave's loads complete in issue order, so the
  // panel loads issued after them do not delay the rotation.
  const int cql = tid % NQL, rsl = tid / NQL;
  u32x4 pl[NL];
#pragma unroll
  for (int u = 0; u < NL; u++) pl[u] = load16(Prs, ((rsl + RSL * u) * D + 4 * cql) * 4);
  float xv[(GR * D + NT - 1) / NT];
#pragma unroll
  for (int u = 0; u < (GR * D + NT - 1) / NT; u++) {
    const int e = min(tid + u * NT, GR * D - 1);  // clamped: the load needs no branch
    if constexpr (APPEND)
      xv[u] = e < G * D ? load_elem<DT>(p.q, q0 * D + e)
                        : load_elem<DT>(p.k_new, head * D + (e - G * D));
    else
      xv[u] = load_elem<DT>(p.q, q0 * D + e);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the panel loads

  // ---- 1a. two panel batches in flight during the rotation
  const int c = tid % LPT, tl = tid / LPT;
  const Rsrc prs = make_rsrc(static_cast<const char*>(p.kcache) +
                                 head * sh.kl.head_elems * (size_t)Elem<DT>::kBytes,
                             (uint32_t)((size_t)sh.S_cap * LPT * 16));
  const int n_pass = (S + TPP - 1) / TPP;
  auto issue = [&](u32x4 (&x)[NB], int pass0) {
#pragma unroll
    for (int it = 0; it < NB; it++) {
      const int t = (pass0 + it) * TPP + tl;
      const uint32_t off = t < Ss ? ((uint32_t)t * LPT + c) * 16 : kOutOfRange;
      // a unit with a helper keeps its panel in L2 for the helper's second read
      x[it] = KEEP ? load16(prs, off) : load16_stream(prs, off);
    }
  };
  u32x4 xa[NB], xb[NB];
  issue(xa, 0);
  issue(xb, NB);

#pragma unroll
  for (int u = 0; u < (GR * D + NT - 1) / NT; u++) {
    const int e = tid + u * NT;
    if (e < GR * D) xq[e / D][e % D] = xv[u];
  }
  if (G == 1) select_clear<NT>(ssm);  // the histogram fills while scoring
  __syncthreads();
  {
    float a[GR][4];
#pragma unroll
    for (int h = 0; h < GR; h++)
#pragma unroll
      for (int cc = 0; cc < 4; cc++) a[h][cc] = 0.f;
#pragma unroll
    for (int u = 0; u < NL; u++) {
      float f[4];
      unpack16<F32>(pl[u], f);
#pragma unroll
      for (int h = 0; h < GR; h++) {
        const float x = xq[h][rsl + RSL * u];
#pragma unroll
        for (int cc = 0; cc < 4; cc++) a[h][cc] = fmaf(x, f[cc], a[h][cc]);
      }
    }
    // lanes of one column quad are NQL apart within the wave
#pragma unroll
    for (int o = NQL; o < 64; o <<= 1)
#pragma unroll
      for (int h = 0; h < GR; h++)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) a[h][cc] += __shfl_xor(a[h][cc], o, 64);
    if (lane < NQL)
#pragma unroll
      for (int h = 0; h < GR; h++)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) qpart[wave][h][4 * cql + cc] = a[h][cc];
  }
  __syncthreads();
  for (int e = tid; e < GR * DP; e += NT) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; w++) s += qpart[w][e / DP][e % DP];
    if (!APPEND || e < G * DP) {
      qs[e / DP][e % DP] = s;
    } else {  // panel coordinate of the new key: stored, and kept as stored
      store_elem<DT>(p.kcache, head * sh.kl.head_elems + (size_t)(S - 1) * DP + e % DP, s);
      kn[e % DP] = stored_value<DT>(s);
    }
  }
  __syncthreads();

  LOKI_STAMP(g_stamps_fused, 1);
  __builtin_amdgcn_s_setprio(0);
  // ---- 1b. low-dim scores of every token into LDS.  Single head: the
  // scores of the first batch fix a provisional binning range, the select
  // histogram is built as the remaining scores are produced (clamped linear
  // bins stay monotone, whatever the range).  Several heads: the exact range
  // is tracked and the histograms are built after scoring.
  {
    float qv[G][E];
#pragma unroll
    for (int h = 0; h < G; h++) {
      lo[h] = INFINITY;
      hi[h] = -INFINITY;
#pragma unroll
      for (int e = 0; e < E; e++) qv[h][e] = qs[h][c * E + e];  // c*E < DP == d
    }
    if constexpr (APPEND) {
      // score of the new token from its stored panel coordinates, summed as
      // the stream sums a row: lane (h, cl) of wave 0 forms the partial over
      // coordinates [cl*E, cl*E + E), group_sum adds the LPT partials pairwise
      // (the reduce-scatter of the single-head stream adds the same pairs)
      if (wave == 0) {
        const int h = min(lane / LPT, G - 1), cl = lane % LPT;
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) a = fmaf(qs[h][cl * E + e], kn[cl * E + e], a);
        a = group_sum<LPT>(a);
        if (lane < G * LPT && cl == 0) {
          if constexpr (G == 1)
            sk[S - 1] = order_key_nz(a + 0.f);
          else
            sc[h * S + S - 1] = a;
#pragma unroll
          for (int hh = 0; hh < G; hh++)
            if (hh == h) {
              lo[hh] = fminf(lo[hh], a);
              hi[hh] = fmaxf(hi[hh], a);
            }
        }
      }
    }
    auto consume = [&](const u32x4 (&x)[NB], int pass0, bool hist) {
      if constexpr (G == 1 && LPT == 4 && NB % 4 == 0) {
        // Each lane's partial dot product for each pass of the batch, then a
        // reduce-scatter over groups of 4 passes: lane c of a quad ends with
        // the whole score of pass (group + c) and stores and bins it itself.
        // The pairs are added as in group_sum<4>, so the scores are the same.
        float a[NB];
#pragma unroll
        for (int it = 0; it < NB; it++) {
          float f[E];
          unpack16<DT>(x[it], f);
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < E; e++) acc = fmaf(qv[0][e], f[e], acc);
          a[it] = acc;
        }
        const bool b0 = (c & 1) != 0, b1 = (c & 2) != 0;
#pragma unroll
        for (int g0 = 0; g0 < NB; g0 += 4) {
          const float u0 = (b0 ? a[g0 + 1] : a[g0]) + dpp_f<0xB1>(b0 ? a[g0] : a[g0 + 1]);
          const float u1 = (b0 ? a[g0 + 3] : a[g0 + 2]) + dpp_f<0xB1>(b0 ? a[g0 + 2] : a[g0 + 3]);
          const float r = (b1 ? u1 : u0) + dpp_f<0x4E>(b1 ? u0 : u1);
          const int t = (pass0 + g0 + c) * TPP + tl;
          if (t < Ss) {
            lo[0] = fminf(lo[0], r);
            hi[0] = fmaxf(hi[0], r);
            sk[t] = order_key_nz(r + 0.f);  // + 0 turns -0 into +0
            if (hist) atomicAdd(&ssm.hist[lin_bin(r, blo, bscale)], 1u);
          }
        }
        return;
      }
#pragma unroll
      for (int it = 0; it < NB; it++) {
        float f[E];
        unpack16<DT>(x[it], f);
        const int t = (pass0 + it) * TPP + tl;
#pragma unroll
        for (int h = 0; h < G; h++) {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < E; e++) a = fmaf(qv[h][e], f[e], a);
          a = group_sum<LPT>(a);
          if (t < Ss) {
            lo[h] = fminf(lo[h], a);
            hi[h] = fmaxf(hi[h], a);
            if (c == (h % LPT)) {
              if constexpr (G == 1) {
                sk[t] = order_key_nz(a + 0.f);
                if (hist) atomicAdd(&ssm.hist[lin_bin(a, blo, bscale)], 1u);
              } else {
                sc[h * S + t] = a;
              }
            }
          }
        }
      }
    };
    consume(xa, 0, false);
    if (G == 1) {
      // provisional range from the first batch of scores, then their histogram
      const float l0 = -wave_max(-lo[0]), h0 = wave_max(hi[0]);
      if (lane == 0) {
        rng[0][wave][0] = l0;
        rng[1][wave][0] = h0;
      }
      __syncthreads();
      blo = rng[0][0][0];
      float bhi = rng[1][0][0];
#pragma unroll
      for (int w = 1; w < NW; w++) {
        blo = fminf(blo, rng[0][w][0]);
        bhi = fmaxf(bhi, rng[1][w][0]);
      }
      bscale = bin_scale(blo, bhi);
      for (int t = tid; t < min(S, NB * TPP); t += NT)
        atomicAdd(&ssm.hist[lin_bin(key_score(sk[t]), blo, bscale)], 1u);
      if (APPEND && tid == 0 && S - 1 >= NB * TPP)  // the new token, past the first batch
        atomicAdd(&ssm.hist[lin_bin(key_score(sk[S - 1]), blo, bscale)], 1u);
    }
    // every batch is issued, also past the end (those loads are out of range:
    // zeros, no memory access), so that the loads in flight are the same on
    // every path and each use waits only for its own batch; the scheduling
    // barriers keep each batch's use after the issue of the next one
    issue(xa, 2 * NB);
    __builtin_amdgcn_sched_barrier(0);
    consume(xb, NB, true);
    issue(xb, 3 * NB);
    __builtin_amdgcn_sched_barrier(0);
    for (int pass = 2 * NB; pass < n_pass; pass += 2 * NB) {
      consume(xa, pass, true);
      issue(xa, pass + 2 * NB);
      __builtin_amdgcn_sched_barrier(0);
      consume(xb, pass + NB, true);
      issue(xb, pass + 3 * NB);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  };
  if (paired)
    phase01(std::true_type{});
  else
    phase01(std::false_type{});
  if (G > 1) {
#pragma unroll
    for (int h = 0; h < G; h++) {
      lo[h] = -wave_max(-lo[h]);
      hi[h] = wave_max(hi[h]);
    }
    if (lane == 0)
#pragma unroll
      for (int h = 0; h < G; h++) {
        rng[0][wave][h] = lo[h];
        rng[1][wave][h] = hi[h];
      }
  }

  LOKI_STAMP(g_stamps_fused, 2);
  __builtin_amdgcn_s_setprio(3);
  // ---- 0'. the rest of the rotation: its P loads stay in flight through the top-k
  const int cqr = tid % 32, rsr = tid / 32;
  u32x4 pr[NR];
#pragma unroll
  for (int u = 0; u < NR; u++)
    pr[u] = load16(Prs, cqr < NQR ? ((rsr + RSR * u) * D + DP + 4 * cqr) * 4 : kOutOfRange);
  // the new value row, copied as raw elements (stored with the rest of the key row)
  using Raw = typename std::conditional<Elem<DT>::kBytes == 4, unsigned, unsigned short>::type;
  Raw vraw = 0;
  if constexpr (APPEND) vraw = static_cast<const Raw*>(p.v_new)[head * D + min(tid, D - 1)];
  __syncthreads();
  LOKI_STAMP(g_stamps_fused, 5);

  // ---- 2. top-k of each head's scores, from LDS.  Single head: the order
  // keys go to registers and select_keys (select_core.h) writes the selected
  // tokens in ascending order with their keys, which the attention reads as
  // the partial logits.  Several heads: block_select per head.
  unsigned* skey = reinterpret_cast<unsigned*>(slow);  // [k] (single head)
  auto rotate_rest = [&]() {  // qpart[w][h][DP:D] from the P loads in flight
    float a[GR][4];
#pragma unroll
    for (int h = 0; h < GR; h++)
#pragma unroll
      for (int cc = 0; cc < 4; cc++) a[h][cc] = 0.f;
#pragma unroll
    for (int u = 0; u < NR; u++) {
      float f[4];
      unpack16<F32>(pr[u], f);
#pragma unroll
      for (int h = 0; h < GR; h++) {
        const float x = xq[h][rsr + RSR * u];
#pragma unroll
        for (int cc = 0; cc < 4; cc++) a[h][cc] = fmaf(x, f[cc], a[h][cc]);
      }
    }
#pragma unroll
    for (int h = 0; h < GR; h++)
#pragma unroll
      for (int cc = 0; cc < 4; cc++) a[h][cc] += __shfl_xor(a[h][cc], 32, 64);
    if (lane < 32 && cqr < NQR)
#pragma unroll
      for (int h = 0; h < GR; h++)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) qpart[wave][h][DP + 4 * cqr + cc] = a[h][cc];
  };
  auto reduce_rest = [&]() {  // qs[h][DP:D] = sum over the waves of qpart
    for (int e = tid; e < GR * (D - DP); e += NT) {
      const int h = e / (D - DP), j = DP + e % (D - DP);
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; w++) s += qpart[w][h][j];
      if (!APPEND || h < G)
        qs[h][j] = s;
      else  // the rest of the new key's row
        store_elem<DT>(p.kcache, head * sh.kl.head_elems + sh.kl.rest_off +
                                     (size_t)(S - 1) * (D - DP) + (j - DP), s);
    }
    if constexpr (APPEND) {
      if (tid < D) static_cast<Raw*>(p.vcache)[(head * sh.S_cap + (size_t)(S - 1)) * D + tid] = vraw;
      // the attention's gathers may read row S-1: every store of this wave
      // (key row, value row) is complete before the barrier that follows
      wait_stores();
    }
  };
  {
    if constexpr (G == 1) {
      // ---- 0''. the rest of the rotation runs inside the selection: the
      // partial sums once the threshold group is known (the P loads have
      // arrived by then), their reduction after the barriers that follow
      KeyRow<NT, KREG> row(sk, S);  // elements past the row: key 0 (select_keys)
      select_keys<NT, KREG>(row, k, sidx, skey, ssm, blo, bscale, ssm.whist, [&](int i) {
        LOKI_STAMP(g_stamps_fused, 6 + i);
        if (i == 0) rotate_rest();
        if (i == 1) reduce_rest();
      });
      __syncthreads();
    } else {
      for (int h = 0; h < G; h++) {
        float l0 = rng[0][0][h], h0 = rng[1][0][h];
#pragma unroll
        for (int w = 1; w < NW; w++) {
          l0 = fminf(l0, rng[0][w][h]);
          h0 = fmaxf(h0, rng[1][w][h]);
        }
        const float* row = sc + h * S;
        auto load_score = [&](int i) -> float { return i < S ? row[i] : 0.f; };
        block_select<NT, KREG>(load_score, S, k, sidx + h * k, slow + h * k, ssm, true, l0,
                                     h0);
        __syncthreads();
      }
      // ---- 0''. finish the rotation: qs[h][DP:D]
      rotate_rest();
      __syncthreads();
      reduce_rest();
      __syncthreads();
    }
  }

  LOKI_STAMP(g_stamps_fused, 3);
  __builtin_amdgcn_s_setprio(0);
  // ---- 3. exact attention over the selected tokens of each head
  // (the index sets, when asked for, are written after it: off its critical path)
  auto write_idx = [&]() {
    if (p.idx_out && !helper)
      for (int e = tid; e < G * k; e += NT) p.idx_out[q0 * k + e] = sidx[e];
  };
  // rows [r0, r0 + nr) of head h's selected list (single head: the partial
  // logits as order keys, rows read once; several heads: as floats, rows
  // kept in L2 for the group's other heads)
  auto attend = [&](int h, int r0, int nr, float& M, float& L, float& A) {
    if constexpr (G == 1)
      block_attend<DT, D, NT, true, kFusedRowsPerBatch, false, true>(
          qs[0], p.scale_log2, sidx + r0, skey + r0, nr, p.kcache, p.vcache, head, sh, asm_, M,
          L, A);
    else
      block_attend<DT, D, NT, true, kFusedRowsPerBatch, false, false>(
          qs[h], p.scale_log2, sidx + h * k + r0, slow + h * k + r0, nr, p.kcache, p.vcache,
          head, sh, asm_, M, L, A);
  };
  if (paired) {
    // owner: rows [0, k0); helper: rows [k0, k).  Partials (M, L, A[D]) of
    // pair j: owner's at help_part[2j], helper's at help_part[2j+1].
    const int r0 = helper ? p.k0 : 0, nr = helper ? k - p.k0 : p.k0;
    float M, L, A;
    attend(0, r0, nr, M, L, A);
    float* mine = p.help_part + ((size_t)pair * 2 + (helper ? 1 : 0)) * (D + 2);
    const float* other = p.help_part + ((size_t)pair * 2 + (helper ? 0 : 1)) * (D + 2);
    if (tid < D) st_coherent(mine + 2 + tid, A);
    if (tid == 0) {
      st_coherent(mine, M);
      st_coherent(mine + 1, L);
    }
    wait_stores();
    __syncthreads();
    if (tid == 0) {
      later = __hip_atomic_exchange(p.help_flag + pair, p.tag, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == p.tag;
      // both halves are in: the flag goes back to 0, so that the next launch
      // on this workspace -- also a replay of a captured one, whose tag is the
      // captured tag -- finds no tag there
      if (later)
        __hip_atomic_store(p.help_flag + pair, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (later && tid < D) {
      const float oM = ld_coherent(other), oL = ld_coherent(other + 1);
      const float oA = ld_coherent(other + 2 + tid);
      // always the owner's half first: the result does not depend on which merges
      store_out(p.out, head * D + tid,
                helper ? combine_partials(oM, oL, oA, M, L, A)
                       : combine_partials(M, L, A, oM, oL, oA),
                sh.odt);
    }
    write_idx();
    LOKI_STAMP(g_stamps_fused, 4);
    return;
  }
  for (int h = 0; h < G; h++) {
    float M, L, A;
    attend(h, 0, k, M, L, A);
    if (tid < D) store_out(p.out, (q0 + h) * D + tid, A / L, sh.odt);
    __syncthreads();  // asm_ is reused by the next head
  }
  write_idx();
  LOKI_STAMP(g_stamps_fused, 4);
}

template <int DT, int D, int LPT, int NT, bool APPEND>
hipError_t launch_nt(const FusedParams& p, size_t dyn, hipStream_t st) {
  const dim3 grid((unsigned)(p.n_units + p.n_help));
  switch (p.sh.g) {
    case 1: fused_kernel<DT, D, LPT, 1, NT, APPEND><<<grid, NT, dyn, st>>>(p); break;
    case 2: fused_kernel<DT, D, LPT, 2, NT, APPEND><<<grid, NT, dyn, st>>>(p); break;
    default: fused_kernel<DT, D, LPT, 4, NT, APPEND><<<grid, NT, dyn, st>>>(p); break;
  }
  return hipGetLastError();
}

template <int DT, int D, int LPT, int NT>
hipError_t launch_append(const FusedParams& p, size_t dyn, hipStream_t st) {
  return p.k_new ? launch_nt<DT, D, LPT, NT, true>(p, dyn, st)
                 : launch_nt<DT, D, LPT, NT, false>(p, dyn, st);
}

template <int DT, int D, int LPT>
hipError_t launch_lpt(const FusedParams& p, size_t dyn, hipStream_t st) {
  return p.threads == 512 ? launch_append<DT, D, LPT, 512>(p, dyn, st)
                          : launch_append<DT, D, LPT, 256>(p, dyn, st);
}

template <int DT>
hipError_t launch_dt(const FusedParams& p, size_t dyn, hipStream_t st) {
  const int lpt = p.sh.dp * Elem<DT>::kBytes / 16;
  return lpt == 4 ? launch_lpt<DT, 128, 4>(p, dyn, st) : launch_lpt<DT, 128, 8>(p, dyn, st);
}

size_t dyn_bytes(const Shape& sh, int k) {
  return (size_t)sh.g * ((size_t)sh.S * 4 + (size_t)k * 8);
}

}  // namespace

bool fused_supported(const Shape& sh, int d, int k) {
  const int eb = sh.dtype == F32 ? 4 : 2;
  const int lpt = sh.dp * eb / 16;
  return d == sh.dp && sh.D == 128 && (lpt == 4 || lpt == 8) &&
         (sh.g == 1 || sh.g == 2 || sh.g == 4) && sh.S <= kFusedMaxS &&
         dyn_bytes(sh, k) <= kFusedDynBytes;
}

hipError_t launch_fused(const FusedParams& p, hipStream_t st) {
  const size_t dyn = dyn_bytes(p.sh, p.k);
  switch (p.sh.dtype) {
    case F32: return launch_dt<F32>(p, dyn, st);
    case F16: return launch_dt<F16>(p, dyn, st);
    default: return launch_dt<BF16>(p, dyn, st);
  }
}

}  // namespace loki

LOKI_STAMP_EXPORT(loki_phase_stamps_fused, loki::g_stamps_fused);
