// Approximate (low-dimensional) attention scores of every cached token.
//
// Loki (briefgpt.xyz abstract; poster page "Visual Insights", Figure 1 right):
// tokens are ranked by attention scores computed from the leading principal
// components only.  s[b,h,t] = sum_{j<d} qr[b,h,j] * krot[b,kv,t,j].
//
// Fast path (d <= dp): the leading dp coordinates of all tokens of one
// (batch, KV head) are one contiguous panel, so a workgroup streams a tile of
// it with 16-byte loads, LPT lanes per token (LPT = dp*elem/16), every lane
// holding the matching fp32 slice of qr for each query head of the KV group;
// the LPT partial dot products are summed with DPP.  One pass over the panel
// serves all g query heads of a GQA group.  In a decode step the kernel can
// also rotate the query itself (head_dim 128, staged tiles): each workgroup
// forms the panel coordinates of its g rotated query rows from P's leading
// columns while its first panel batches are in flight, and the first tile of
// each (b, kv) also forms the remaining coordinates and writes the rotated
// rows for the attention -- one launch fewer per step.  With an append the
// last tile of each (b, kv) rotates the new key as one more row, writes row
// S-1 of both caches (the attention, a later launch, reads it there) and
// replaces the new token's score by the one formed from the rounded row it
// wrote, with the stream's per-lane partials and pairwise sums.  With four lanes per token and
// g <= 4, a tile's scores are staged in LDS and written at the end of the
// tile in 16-byte stores: writes interleaved with the panel stream cost the
// read stream more than one burst of whole lines.
#include "loki_internal.h"

namespace loki {

namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreBatch = 8;  // 16-byte loads per lane per batch; two batches in flight
// scores of one tile staged in LDS (all g heads): groups of four heads take
// 2048-token tiles (one round of workgroups at the grouped-query shapes)
constexpr int stage_scores(int g) { return g == 4 ? 8192 : 4096; }

// Tiles whose scores go through LDS: four lanes per token, g in {1, 2, 4}.
template <int LPT, int G>
constexpr bool kStaged = LPT == 4 && (G == 1 || G == 2 || G == 4);

// One workgroup streams a tile of p.tile_tokens tokens of one (b, kv) panel.
template <int DT, int LPT, int G, bool ROT>
__global__ __launch_bounds__(kScoreThreads) void score_panel_kernel(ScoreParams p) {
  constexpr bool STAGE = kStaged<LPT, G>;
  static_assert(!ROT || STAGE, "the rotating variant is a staged one");
  __shared__ __align__(16) float stage[STAGE ? stage_scores(G) : 1];  // [G][tile_tokens]
  constexpr int E = Elem<DT>::kPerVec;
  constexpr int TPP = kScoreThreads / LPT;  // tokens per pass
  constexpr int NB = kScoreBatch;
  const Shape& sh = p.sh;

  const int tile = blockIdx.x % p.n_tiles;
  const size_t head = blockIdx.x / p.n_tiles;  // b * Hkv + kv
  const int b = (int)(head / sh.Hkv), kv = (int)(head % sh.Hkv);
  const int c = threadIdx.x % LPT;
  const int tl = threadIdx.x / LPT;
  const int t0 = tile * p.tile_tokens;
  const int t_end = min(sh.S, t0 + p.tile_tokens);
  const int n_pass = (t_end - t0 + TPP - 1) / TPP;

  // the panel of this (b, kv): S_cap rows of LPT*16 bytes; tokens past the
  // tile read as zeros
  const Rsrc prs = make_rsrc(static_cast<const char*>(p.kcache) +
                                 head * sh.kl.head_elems * (size_t)Elem<DT>::kBytes,
                             (uint32_t)((size_t)sh.S_cap * LPT * 16));
  auto issue = [&](u32x4 (&x)[NB], int pass0) {
#pragma unroll
    for (int it = 0; it < NB; it++) {
      const int t = t0 + (pass0 + it) * TPP + tl;
      x[it] = load16_stream(prs, t < t_end ? ((uint32_t)t * LPT + c) * 16 : kOutOfRange);
    }
  };
  // the rotation (ROT): q rows staged as fp32, per-wave partial sums
  constexpr int RD = 128;                              // head_dim of the rotating variant
  constexpr int DP = LPT * 16 / Elem<DT>::kBytes;      // panel width
  constexpr int NW = kScoreThreads / 64;
  constexpr int NQL = DP / 4, RSL = kScoreThreads / NQL, NL = RD / RSL;
  constexpr int NXV = ROT ? ((G + 1) * RD + kScoreThreads - 1) / kScoreThreads : 1;
  __shared__ float xq[ROT ? G + 1 : 1][RD];          // query rows, then the new key
  // per-wave partial sums of the rotation: they live in the stage, which
  // holds no scores before the stream starts or after the tile is written
  static_assert(!ROT || NW * (G + 1) * RD <= stage_scores(G), "partials fit the stage");
  auto qpart = reinterpret_cast<float (*)[G + 1][RD]>(stage);
  __shared__ float qs[ROT ? G : 1][DP];
  __shared__ float kn[ROT ? DP : 1];                  // new key's panel coordinates as stored
  const size_t q0 = (size_t)b * sh.Hq + (size_t)kv * G;  // first query row of the group
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool last = ROT && p.k_new != nullptr && t_end == sh.S;  // this tile appends token S-1
  // The rotation's loads go out before the panel batches: a wave's loads
  // complete in issue order, so the rotation does not wait for the panel.
  const int cql = tid % NQL, rsl = tid / NQL;
  u32x4 pl[ROT ? NL : 1];
  float xv[NXV];
  if constexpr (ROT) {
    const Rsrc Prs = make_rsrc(p.P + (size_t)kv * RD * RD, (uint32_t)(RD * RD * 4));
#pragma unroll
    for (int u = 0; u < NL; u++) pl[u] = load16(Prs, ((rsl + RSL * u) * RD + 4 * cql) * 4);
#pragma unroll
    for (int u = 0; u < NXV; u++) {
      const int e = tid + u * kScoreThreads;  // query rows, then the new key's row
      // (both offsets are clamped into their rows: every lane's address is valid)
      xv[u] = e < G * RD ? load_elem<DT>(p.q, q0 * RD + min(e, G * RD - 1))
                         : (last ? load_elem<DT>(p.k_new, head * RD + min(max(e - G * RD, 0), RD - 1))
                                 : 0.f);
    }
  }
  u32x4 xa[NB], xb[NB];
  issue(xa, 0);
  issue(xb, NB);
  if constexpr (ROT) {
    // qs[h][0:DP] = q[h] . P[kv][:, 0:DP]: thread = (column quad, row slot)
#pragma unroll
    for (int u = 0; u < NXV; u++) {
      const int e = tid + u * kScoreThreads;
      if (e < (G + 1) * RD) xq[e / RD][e % RD] = xv[u];
    }
    __syncthreads();
    float a[G][4];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
      for (int cc = 0; cc < 4; cc++) a[h][cc] = 0.f;
#pragma unroll
    for (int u = 0; u < NL; u++) {
      float f[4];
      unpack16<F32>(pl[u], f);
#pragma unroll
      for (int h = 0; h < G; h++) {
        const float x = xq[h][rsl + RSL * u];
#pragma unroll
        for (int cc = 0; cc < 4; cc++) a[h][cc] = fmaf(x, f[cc], a[h][cc]);
      }
    }
    // lanes of one column quad are NQL apart within the wave
#pragma unroll
    for (int o = NQL; o < 64; o <<= 1)
#pragma unroll
      for (int h = 0; h < G; h++)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) a[h][cc] += __shfl_xor(a[h][cc], o, 64);
    if (lane < NQL)
#pragma unroll
      for (int h = 0; h < G; h++)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) qpart[wave][h][4 * cql + cc] = a[h][cc];
    if (last) {  // the new key's panel coordinates, from the same P loads
      float ak[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NL; u++) {
        float f[4];
        unpack16<F32>(pl[u], f);
        const float x = xq[G][rsl + RSL * u];
#pragma unroll
        for (int cc = 0; cc < 4; cc++) ak[cc] = fmaf(x, f[cc], ak[cc]);
      }
#pragma unroll
      for (int o = NQL; o < 64; o <<= 1)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) ak[cc] += __shfl_xor(ak[cc], o, 64);
      if (lane < NQL)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) qpart[wave][G][4 * cql + cc] = ak[cc];
    }
    __syncthreads();
    for (int e = tid; e < G * DP; e += kScoreThreads) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; w++) s += qpart[w][e / DP][e % DP];
      qs[e / DP][e % DP] = s;
    }
    if (last)
      for (int j = tid; j < DP; j += kScoreThreads) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NW; w++) s += qpart[w][G][j];
        store_elem<DT>(p.kcache_w, head * sh.kl.head_elems + (size_t)(sh.S - 1) * DP + j, s);
        kn[j] = stored_value<DT>(s);
      }
    __syncthreads();
  }

  // qr slices (read after the first panel loads are issued, so that both are
  // in flight)
  float qv[G][E];
#pragma unroll
  for (int h = 0; h < G; h++) {
#pragma unroll
    for (int e = 0; e < E; e++) {
      const int j = c * E + e;  // < dp <= D: always inside the row
      float v;
      if constexpr (ROT)
        v = qs[h][j];
      else
        v = p.qr[(q0 + h) * sh.D + j];
      qv[h][e] = (j < p.d) ? v : 0.f;
    }
  }

  float* srow = p.scores + ((size_t)b * sh.Hq + (size_t)kv * G) * sh.S;
  auto consume = [&](const u32x4 (&x)[NB], int pass0) {
    if constexpr (G == 1 && LPT == 4 && NB % 4 == 0) {
      // reduce-scatter over groups of 4 passes: lane c of a quad ends with the
      // whole score of pass (group + c) (pairs added as in group_sum<4>)
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
        const int t = t0 + (pass0 + g0 + c) * TPP + tl;
        if (t < t_end) stage[t - t0] = r;
      }
      return;
    }
    if constexpr ((G == 4 || G == 2) && LPT == 4) {
      // reduce-scatter over the heads: after the pair and quad exchanges
      // lane c holds the whole score of head c (G = 4) or of head c % 2
      // (G = 2, stored by lanes 0 and 1)
      const bool b0 = (c & 1) != 0, b1 = (c & 2) != 0;
#pragma unroll
      for (int it = 0; it < NB; it++) {
        float f[E];
        unpack16<DT>(x[it], f);
        float a[G];
#pragma unroll
        for (int h = 0; h < G; h++) {
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < E; e++) acc = fmaf(qv[h][e], f[e], acc);
          a[h] = acc;
        }
        float r;
        if constexpr (G == 4) {
          const float u0 = (b0 ? a[1] : a[0]) + dpp_f<0xB1>(b0 ? a[0] : a[1]);
          const float u1 = (b0 ? a[3] : a[2]) + dpp_f<0xB1>(b0 ? a[2] : a[3]);
          r = (b1 ? u1 : u0) + dpp_f<0x4E>(b1 ? u0 : u1);
        } else {
          const float u = (b0 ? a[1] : a[0]) + dpp_f<0xB1>(b0 ? a[0] : a[1]);
          r = u + dpp_f<0x4E>(u);
        }
        const int t = t0 + (pass0 + it) * TPP + tl;
        if (t < t_end && c < G) stage[c * p.tile_tokens + (t - t0)] = r;
      }
      return;
    }
#pragma unroll
    for (int it = 0; it < NB; it++) {
      float f[E];
      unpack16<DT>(x[it], f);
      float s[G];
#pragma unroll
      for (int h = 0; h < G; h++) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) a = fmaf(qv[h][e], f[e], a);
        s[h] = group_sum<LPT>(a);
      }
      const int t = t0 + (pass0 + it) * TPP + tl;
      if (t < t_end) {
#pragma unroll
        for (int h = 0; h < G; h++)
          if (c == (h % LPT)) srow[(size_t)h * sh.S + t] = s[h];
      }
    }
  };
  for (int pass = 0; pass < n_pass; pass += 2 * NB) {
    consume(xa, pass);
    if (pass + 2 * NB < n_pass) issue(xa, pass + 2 * NB);
    consume(xb, pass + NB);
    if (pass + 3 * NB < n_pass) issue(xb, pass + 3 * NB);
  }
  if constexpr (STAGE) {
    __syncthreads();  // every stream store of this tile's scores is in LDS
    if constexpr (ROT) {
      if (last) {
        // the new token's score from its stored panel coordinates (the
        // stream read the row before this kernel's store may have landed):
        // lane (h, cl) of wave 0 forms the partial over [cl*E, cl*E + E),
        // group_sum adds the four partials pairwise (the stream's
        // reduce-scatter adds the same pairs)
        if (wave == 0) {
          const int h = min(lane / LPT, G - 1), cl = lane % LPT;
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < E; e++) {
            const int j = cl * E + e;
            acc = fmaf(j < p.d ? qs[h][j] : 0.f, kn[j], acc);
          }
          acc = group_sum<LPT>(acc);
          if (lane < G * LPT && cl == 0) stage[h * p.tile_tokens + (sh.S - 1 - t0)] = acc;
        }
        __syncthreads();
      }
    }
    // the tile's scores, head by head: 16-byte stores where the row allows
    // (t0 is a multiple of the pass step, so it is 16-byte aligned when S is
    // a multiple of 4), scalar stores for the rest
    const int n = t_end - t0;
    const int n4 = (sh.S % 4 == 0) ? n / 4 * 4 : 0;
#pragma unroll
    for (int h = 0; h < G; h++) {
      float* dst = srow + (size_t)h * sh.S + t0;
      const float* src = stage + h * p.tile_tokens;
      for (int e = threadIdx.x * 4; e < n4; e += kScoreThreads * 4)
        *reinterpret_cast<float4*>(dst + e) = *reinterpret_cast<const float4*>(src + e);
      for (int e = n4 + threadIdx.x; e < n; e += kScoreThreads) dst[e] = src[e];
    }
    if constexpr (ROT) __syncthreads();  // the stage is read out: the partials may reuse it
  }
  if constexpr (ROT) {
    if (last) {
      // the rest of the new key's row and its value row
      constexpr int NQR = (RD - DP) / 4, RSR = kScoreThreads / 32, NR = RD / RSR;
      const int cqr = tid % 32, rsr = tid / 32;
      const Rsrc Prs = make_rsrc(p.P + (size_t)kv * RD * RD, (uint32_t)(RD * RD * 4));
      u32x4 pr[NR];
#pragma unroll
      for (int u = 0; u < NR; u++)
        pr[u] = load16(Prs, cqr < NQR ? ((rsr + RSR * u) * RD + DP + 4 * cqr) * 4 : kOutOfRange);
      float ak[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NR; u++) {
        float f[4];
        unpack16<F32>(pr[u], f);
        const float x = xq[G][rsr + RSR * u];
#pragma unroll
        for (int cc = 0; cc < 4; cc++) ak[cc] = fmaf(x, f[cc], ak[cc]);
      }
#pragma unroll
      for (int cc = 0; cc < 4; cc++) ak[cc] += __shfl_xor(ak[cc], 32, 64);
      if (lane < 32 && cqr < NQR)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) qpart[wave][G][DP + 4 * cqr + cc] = ak[cc];
      __syncthreads();
      for (int j = DP + tid; j < RD; j += kScoreThreads) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NW; w++) s += qpart[w][G][j];
        store_elem<DT>(p.kcache_w, head * sh.kl.head_elems + sh.kl.rest_off +
                                       (size_t)(sh.S - 1) * (RD - DP) + (j - DP), s);
      }
      for (int j = tid; j < RD; j += kScoreThreads)
        copy_elem<DT>(p.vcache_w, (head * sh.S_cap + (size_t)(sh.S - 1)) * RD + j, p.v_new,
                      head * RD + j);
    }
    // the first tile of each (b, kv): the remaining coordinates,
    // qs[h][DP:RD] = q[h] . P[kv][:, DP:RD] (32 quad slots x 8 row slots), and
    // the rotated rows for the attention
    if (tile == 0) {
      constexpr int NQR = (RD - DP) / 4, RSR = kScoreThreads / 32, NR = RD / RSR;
      static_assert(NQR <= 32, "quad slots");
      const int cqr = tid % 32, rsr = tid / 32;
      const Rsrc Prs = make_rsrc(p.P + (size_t)kv * RD * RD, (uint32_t)(RD * RD * 4));
      u32x4 pr[NR];
#pragma unroll
      for (int u = 0; u < NR; u++)
        pr[u] = load16(Prs, cqr < NQR ? ((rsr + RSR * u) * RD + DP + 4 * cqr) * 4 : kOutOfRange);
      float a[G][4];
#pragma unroll
      for (int h = 0; h < G; h++)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) a[h][cc] = 0.f;
#pragma unroll
      for (int u = 0; u < NR; u++) {
        float f[4];
        unpack16<F32>(pr[u], f);
#pragma unroll
        for (int h = 0; h < G; h++) {
          const float x = xq[h][rsr + RSR * u];
#pragma unroll
          for (int cc = 0; cc < 4; cc++) a[h][cc] = fmaf(x, f[cc], a[h][cc]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; h++)
#pragma unroll
        for (int cc = 0; cc < 4; cc++) a[h][cc] += __shfl_xor(a[h][cc], 32, 64);
      if (lane < 32 && cqr < NQR)
#pragma unroll
        for (int h = 0; h < G; h++)
#pragma unroll
          for (int cc = 0; cc < 4; cc++) qpart[wave][h][DP + 4 * cqr + cc] = a[h][cc];
      __syncthreads();
      for (int e = tid; e < G * RD; e += kScoreThreads) {
        const int h = e / RD, j = e % RD;
        float s;
        if (j < DP) {
          s = qs[h][j];
        } else {
          s = 0.f;
#pragma unroll
          for (int w = 0; w < NW; w++) s += qpart[w][h][j];
        }
        p.qr_out[(q0 + h) * RD + j] = s;
      }
    }
  }
}

// Any d (including d > dp): one thread per token, element loads.
template <int DT>
__global__ __launch_bounds__(kScoreThreads) void score_generic_kernel(ScoreParams p) {
  const Shape& sh = p.sh;
  const int tile = blockIdx.x % p.n_tiles;
  const size_t head = blockIdx.x / p.n_tiles;
  const int b = (int)(head / sh.Hkv), kv = (int)(head % sh.Hkv);
  const int t = tile * kScoreThreads + threadIdx.x;
  if (t >= sh.S) return;
  for (int h = 0; h < sh.g; h++) {
    const size_t qh = (size_t)b * sh.Hq + (size_t)kv * sh.g + h;
    const float* qrow = p.qr + qh * sh.D;
    float a = 0.f;
    for (int j = 0; j < p.d; j++)
      a = fmaf(qrow[j], load_elem<DT>(p.kcache, sh.kl.at(head, (size_t)t, j)), a);
    p.scores[qh * sh.S + t] = a;
  }
}

// Tokens per tile of the panel kernel with LPT lanes per token: up to 4096
// (256 KB of an fp16 panel), smaller when that leaves fewer than two
// workgroups per compute unit (when a tile also writes the scores of several
// heads: four for groups of four heads, whose 2048-token tiles were measured
// faster that way, eight for the other group sizes); multiples of two
// batches; staged tiles hold all g heads' scores of the tile in LDS.
int tile_tokens(const Shape& sh, int lpt) {
  const int step = (kScoreThreads / lpt) * 2 * kScoreBatch;
  const long long units = (long long)sh.B * sh.Hkv;
  const int per_grid = sh.g == 1 ? 512 : (sh.g == 4 ? 1024 : 2048);
  long long want = (long long)sh.S * units / per_grid;
  const bool staged = lpt == 4 && (sh.g == 1 || sh.g == 2 || sh.g == 4);
  const long long cap = staged ? stage_scores(sh.g) / sh.g : 4096;
  want = want < step ? step : (want > cap ? cap : want);
  return (int)((want + step - 1) / step * step);
}

template <int DT, int LPT>
hipError_t launch_lpt(ScoreParams p, hipStream_t st) {
  p.tile_tokens = tile_tokens(p.sh, LPT);
  p.n_tiles = (p.sh.S + p.tile_tokens - 1) / p.tile_tokens;
  const dim3 grid((unsigned)((size_t)p.n_tiles * p.sh.B * p.sh.Hkv));
  if constexpr (LPT == 4) {
    if (p.q) {  // the rotating variant (head_dim 128, g in {1, 2, 4}: checked by the caller)
      switch (p.sh.g) {
        case 1: score_panel_kernel<DT, LPT, 1, true><<<grid, kScoreThreads, 0, st>>>(p); break;
        case 2: score_panel_kernel<DT, LPT, 2, true><<<grid, kScoreThreads, 0, st>>>(p); break;
        default: score_panel_kernel<DT, LPT, 4, true><<<grid, kScoreThreads, 0, st>>>(p); break;
      }
      return hipGetLastError();
    }
  }
  switch (p.sh.g) {
    case 1: score_panel_kernel<DT, LPT, 1, false><<<grid, kScoreThreads, 0, st>>>(p); break;
    case 2: score_panel_kernel<DT, LPT, 2, false><<<grid, kScoreThreads, 0, st>>>(p); break;
    case 4: score_panel_kernel<DT, LPT, 4, false><<<grid, kScoreThreads, 0, st>>>(p); break;
    default: score_panel_kernel<DT, LPT, 8, false><<<grid, kScoreThreads, 0, st>>>(p); break;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(ScoreParams p, hipStream_t st) {
  const int lpt = p.sh.dp * Elem<DT>::kBytes / 16;
  const int g = p.sh.g;
  const bool fast = p.d <= p.sh.dp && (g == 1 || g == 2 || g == 4 || g == 8) &&
                    (lpt == 2 || lpt == 4 || lpt == 8 || lpt == 16);
  if (fast) {
    switch (lpt) {
      case 2: return launch_lpt<DT, 2>(p, st);
      case 4: return launch_lpt<DT, 4>(p, st);
      case 8: return launch_lpt<DT, 8>(p, st);
      default: return launch_lpt<DT, 16>(p, st);
    }
  }
  p.n_tiles = (p.sh.S + kScoreThreads - 1) / kScoreThreads;
  const dim3 grid((unsigned)((size_t)p.n_tiles * p.sh.B * p.sh.Hkv));
  score_generic_kernel<DT><<<grid, kScoreThreads, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

long long score_workgroups_staged(const Shape& sh) {
  const long long n_tiles = (sh.S + tile_tokens(sh, 4) - 1) / tile_tokens(sh, 4);
  return n_tiles * sh.B * sh.Hkv;
}

hipError_t launch_score(const ScoreParams& p, hipStream_t st) {
  switch (p.sh.dtype) {
    case F32: return launch_dt<F32>(p, st);
    case F16: return launch_dt<F16>(p, st);
    default: return launch_dt<BF16>(p, st);
  }
}

}  // namespace loki
