// The whole Loki decode step for one (batch, KV head) in one workgroup.
//
// Loki (poster page, "Visual Insights", Figure 1 right; "TL;DR"; briefgpt.xyz
// abstract): rotate the query into the PCA basis, score every cached token
// with the leading d coordinates, keep the top k, run exact attention with the
// full-dimensional keys of those k tokens.
//
// One launch, no intermediate buffers in HBM: per unit (b, kv) with its g
// query heads,
//  0. the query rows are rotated by P[kv] (P read from L2, coalesced columns,
//     partial sums over row chunks merged in LDS);
//  1. the contiguous leading-dp panel of the unit's keys is streamed with
//     16-byte loads, two batches in flight, and the g score rows kept in LDS;
//  2. block_select (select_core.h) picks each head's top k from LDS;
//  3. block_attend (attend_core.h) gathers the selected key tails and value
//     rows and writes the output rows.
// A decode step becomes one kernel: no launch gaps, no ramp-up/drain between
// phases, and the scores never leave LDS.  Used when d == dp, the unit's g
// score rows fit the LDS budget and S <= 4096.
#include "attend_core.h"
#include "loki_internal.h"
#include "select_core.h"

namespace loki {

namespace {

constexpr int kFusedThreads = 256;
constexpr int kFusedKreg = 16;            // S <= 256 * 16
constexpr int kFusedBatch = 8;            // 16-byte panel loads per lane per batch
constexpr size_t kFusedDynBytes = 36 * 1024;

template <int DT, int D, int LPT, int G>
__global__ __launch_bounds__(kFusedThreads) void fused_kernel(FusedParams p) {
  constexpr int NT = kFusedThreads;
  constexpr int NW = NT / 64;
  constexpr int E = Elem<DT>::kPerVec;
  constexpr int TPP = NT / LPT;           // tokens per pass over the panel
  constexpr int RG = NT / D;              // row chunks of the rotation
  constexpr int NB = kFusedBatch;

  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ SelectSmem<NW> ssm;
  __shared__ AttendSmem<DT, D, NT> asm_;
  __shared__ float xq[G][D];       // query rows, fp32
  __shared__ float qpart[RG][G][D];
  __shared__ float qs[G][D];       // rotated query rows

  const Shape& sh = p.sh;
  const int S = sh.S, k = p.k;
  float* sc = reinterpret_cast<float*>(dyn);        // [G][S]
  int* sidx = reinterpret_cast<int*>(sc + G * S);   // [G][k]
  float* slow = reinterpret_cast<float*>(sidx + G * k);  // [G][k]

  const size_t head = blockIdx.x;  // b * Hkv + kv
  const int b = (int)(head / sh.Hkv), kv = (int)(head % sh.Hkv);
  const int tid = threadIdx.x;
  const size_t q0 = (size_t)b * sh.Hq + (size_t)kv * G;  // first query head of the group

  // ---- 1a. first panel batch in flight before anything else
  const int c = tid % LPT, tl = tid / LPT;
  const Rsrc prs = make_rsrc(static_cast<const char*>(p.kcache) +
                                 head * sh.kl.head_elems * (size_t)Elem<DT>::kBytes,
                             (uint32_t)((size_t)sh.S_cap * LPT * 16));
  const int n_pass = (S + TPP - 1) / TPP;
  auto issue = [&](u32x4 (&x)[NB], int pass0) {
#pragma unroll
    for (int it = 0; it < NB; it++) {
      const int t = (pass0 + it) * TPP + tl;
      x[it] = load16(prs, t < S ? ((uint32_t)t * LPT + c) * 16 : kOutOfRange);
    }
  };
  u32x4 xa[NB], xb[NB];
  issue(xa, 0);

  // ---- 0. rotation of the g query rows: qs[h] = q[h] . P[kv]
  for (int e = tid; e < G * D; e += NT)
    xq[e / D][e % D] = load_elem<DT>(p.q, q0 * D + e);
  __syncthreads();
  {
    // thread (j, rg) loads its D/RG entries of column j of P[kv] at once
    constexpr int NI = D / RG;
    const int j = tid % D, rg = tid / D;
    const float* Pk = p.P + (size_t)kv * D * D + (size_t)rg * NI * D + j;
    float pv[NI];
#pragma unroll
    for (int u = 0; u < NI; u++) pv[u] = Pk[(size_t)u * D];
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; h++) acc[h] = 0.f;
#pragma unroll
    for (int u = 0; u < NI; u++)
#pragma unroll
      for (int h = 0; h < G; h++) acc[h] = fmaf(xq[h][rg * NI + u], pv[u], acc[h]);
#pragma unroll
    for (int h = 0; h < G; h++) qpart[rg][h][j] = acc[h];
  }
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RG; r++) s += qpart[r][e / D][e % D];
    qs[e / D][e % D] = s;
  }
  __syncthreads();

  // ---- 1b. low-dim scores of every token into LDS
  {
    float qv[G][E];
#pragma unroll
    for (int h = 0; h < G; h++)
#pragma unroll
      for (int e = 0; e < E; e++) qv[h][e] = qs[h][c * E + e];  // c*E < dp == d
    auto consume = [&](const u32x4 (&x)[NB], int pass0) {
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
          if (t < S && c == (h % LPT)) sc[h * S + t] = a;
        }
      }
    };
    for (int pass = 0; pass < n_pass; pass += 2 * NB) {
      issue(xb, pass + NB);
      consume(xa, pass);
      if (pass + 2 * NB < n_pass) issue(xa, pass + 2 * NB);
      consume(xb, pass + NB);
    }
  }
  __syncthreads();

  // ---- 2. top-k of each head's scores, from LDS
  for (int h = 0; h < G; h++) {
    const float* row = sc + h * S;
    auto load_score = [&](int i) -> float { return i < S ? row[i] : 0.f; };
    block_select<NT, kFusedKreg>(load_score, S, k, sidx + h * k, slow + h * k, ssm);
    __syncthreads();
  }

  // ---- 3. exact attention over the selected tokens of each head
  for (int h = 0; h < G; h++) {
    float M, L, A;
    block_attend<DT, D, NT, true>(qs[h], p.scale_log2, sidx + h * k, slow + h * k, k,
                                  p.kcache, p.vcache, head, sh, asm_, M, L, A);
    if (tid < D) p.out[(q0 + h) * D + tid] = A / L;
    if (p.idx_out)
      for (int r = tid; r < k; r += NT) p.idx_out[(q0 + h) * k + r] = sidx[h * k + r];
    __syncthreads();  // asm_ is reused by the next head
  }
}

template <int DT, int D, int LPT>
hipError_t launch_lpt(const FusedParams& p, size_t dyn, hipStream_t st) {
  const dim3 grid((unsigned)(p.sh.B * p.sh.Hkv));
  switch (p.sh.g) {
    case 1: fused_kernel<DT, D, LPT, 1><<<grid, kFusedThreads, dyn, st>>>(p); break;
    case 2: fused_kernel<DT, D, LPT, 2><<<grid, kFusedThreads, dyn, st>>>(p); break;
    default: fused_kernel<DT, D, LPT, 4><<<grid, kFusedThreads, dyn, st>>>(p); break;
  }
  return hipGetLastError();
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
         (sh.g == 1 || sh.g == 2 || sh.g == 4) && sh.S <= kFusedThreads * kFusedKreg &&
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
