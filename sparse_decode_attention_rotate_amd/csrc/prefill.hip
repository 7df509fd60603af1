// Bulk projection of prompt keys into the rotated key cache.
//
// Loki (poster page, "Visual Insights", Figure 1 right): keys are kept in the
// basis of the principal components found offline; a decode step appends
// one key projected by P (poster page, "Loki's Computational Cost").  Prefill
// does the same for a whole prompt: krot[b,kv,t,:] = k[b,kv,t,:] . P[kv] for
// t < n_tokens, rounded once to nearest-even into the storage dtype and written
// into the split-panel layout at rows pos + t -- a dense [n_tokens x D] . [D x D] product per
// (b, kv).
//
// fp16 / bf16 keys, D = 128: MFMA 16x16x32 with fp32 accumulation.  The keys
// are exact in their 16-bit type; P is split into parts of that type,
// P = P_1 + P_2 (fp16, of 1024 * P so that the low part stays clear of the
// fp16 subnormals; the factor is a power of two and divides out exactly) or
// P_1 + P_2 + P_3 (bf16), carrying 22 / 24 significant bits like the fp32
// product of the decode-time append.  Each wave owns 32 output coordinates and
// keeps the parts of those columns of P[kv] in registers; a workgroup walks
// tiles of 64 tokens through LDS (key tile in, rounded output tile out, both
// 16-byte chunks), with the next tile's loads in flight during the products.
// fp32 keys and D = 64 use a VALU kernel: a thread keeps one column of P in
// registers and forms that coordinate for a run of tokens staged in LDS.
#include "loki_internal.h"

namespace loki {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kPreThreads = 256;        // VALU kernel
constexpr int kPreTile = 64;            // tokens per LDS tile
constexpr int kPreWaves = 8;            // MFMA kernel: waves per workgroup
constexpr int kPreDepth = 2;            // MFMA kernel: key tiles in flight

template <int DT> struct Split;
template <> struct Split<F16> {
  static constexpr int N = 2;
  static constexpr float kScale = 1024.f;
};
template <> struct Split<BF16> {
  static constexpr int N = 3;
  static constexpr float kScale = 1.f;
};

// x rounded to nearest-even in the 16-bit type: bit pattern; *back = its value
template <int DT>
__device__ __forceinline__ unsigned round16(float x, float* back) {
  if constexpr (DT == F16) {
    const _Float16 h = (_Float16)x;
    *back = (float)h;
    return __builtin_bit_cast(unsigned short, h);
  } else {
    unsigned u = __float_as_uint(x), r;
    if ((u & 0x7fffffffu) > 0x7f800000u) {
      r = (u >> 16) | 0x40u;  // quiet NaN
    } else {
      u += 0x7fffu + ((u >> 16) & 1u);
      r = u >> 16;
    }
    *back = __uint_as_float(r << 16);
    return r;
  }
}

template <int DT>
__device__ __forceinline__ float4_t mfma32(u32x4 a, u32x4 b, float4_t c) {
  if constexpr (DT == F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Operand layout of the 16x16x32 product (64 lanes): lane l supplies row l%16
// of A and column l%16 of B, each at the 8 inner indices 8*(l/16) .. +7 of the
// 32-wide step; result element i of lane l is row 4*(l/16)+i, column l%16.
// NW waves, each owning D/NW output coordinates (CB blocks of 16); DEPTH key
// tiles in flight (register buffers) ahead of the one in LDS.
template <int DT, int NW, int DEPTH, int TPWG>
__global__ __launch_bounds__(64 * NW, 1024 / (64 * NW)) void prefill_mfma_kernel(PrefillParams p) {
  constexpr int D = 128, NS = Split<DT>::N, KSTEPS = D / 32, TB = kPreTile / 16;
  constexpr int NT = 64 * NW, CB = D / (16 * NW), CPT = kPreTile * 16 / NT;  // chunks per thread
  constexpr int RP = D + 8;  // padded LDS row (16-bit elements): 272 bytes
  __shared__ __align__(16) unsigned short kt[kPreTile][RP];
  __shared__ __align__(16) unsigned short ot[kPreTile][RP];

  const Shape& sh = p.sh;
  const size_t head = blockIdx.y;
  const int kv = (int)(head % sh.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane % 16, kg = lane / 16;
  const int col0 = wave * 16 * CB;

  const int t_begin = blockIdx.x * TPWG;
  const int t_end = min(p.n_tokens, t_begin + TPWG);
  const unsigned short* krow =
      static_cast<const unsigned short*>(p.k_rows) + head * (size_t)p.n_tokens * D;
  // a tile = 64 tokens x 16 chunks of 16 bytes; thread tid moves chunks tid + NT*u
  auto load_tile = [&](u32x4 (&x)[CPT], int t0) {
#pragma unroll
    for (int u = 0; u < CPT; u++) {
      const int c = tid + u * NT, t = t0 + c / 16;
      x[u] = t < t_end ? __builtin_nontemporal_load(
                             reinterpret_cast<const u32x4*>(krow + (size_t)t * D + (c % 16) * 8))
                       : u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 xk[DEPTH][CPT];
#pragma unroll
  for (int b = 0; b < DEPTH; b++) load_tile(xk[b], t_begin + b * kPreTile);

  // parts of this wave's columns of P[kv]: bp[s][cb][ks] holds rows
  // 32ks + 8kg .. +7 of column col0 + 16cb + n
  u32x4 bp[NS][CB][KSTEPS];
  {
    const float* P = p.P + (size_t)kv * D * D;
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ks++) {
        unsigned bits[NS][8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
          float r = P[(size_t)(32 * ks + 8 * kg + j) * D + col0 + 16 * cb + n] * Split<DT>::kScale;
#pragma unroll
          for (int s = 0; s < NS; s++) {
            float v;
            bits[s][j] = round16<DT>(r, &v);
            r -= v;
          }
        }
#pragma unroll
        for (int s = 0; s < NS; s++)
          bp[s][cb][ks] = u32x4{bits[s][0] | (bits[s][1] << 16), bits[s][2] | (bits[s][3] << 16),
                                bits[s][4] | (bits[s][5] << 16), bits[s][6] | (bits[s][7] << 16)};
      }
  }

  // one tile: its keys (in registers) through LDS, products, rounded output
  auto tile = [&](u32x4 (&x)[CPT], int t0) {
    // kt is free: every wave passed the previous tile's second barrier after
    // its last read of kt
#pragma unroll
    for (int u = 0; u < CPT; u++) {
      const int c = tid + u * NT;
      *reinterpret_cast<u32x4*>(&kt[c / 16][(c % 16) * 8]) = x[u];
    }
    if (t0 + DEPTH * kPreTile < t_end) load_tile(x, t0 + DEPTH * kPreTile);
    __syncthreads();

    float4_t acc[TB][CB];
#pragma unroll
    for (int tb = 0; tb < TB; tb++)
#pragma unroll
      for (int cb = 0; cb < CB; cb++) acc[tb][cb] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ks++)
#pragma unroll
      for (int tb = 0; tb < TB; tb++) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&kt[16 * tb + n][32 * ks + 8 * kg]);
#pragma unroll
        for (int cb = 0; cb < CB; cb++)
#pragma unroll
          for (int s = 0; s < NS; s++) acc[tb][cb] = mfma32<DT>(a, bp[s][cb][ks], acc[tb][cb]);
      }
    // ot is free: the previous tile's reads of ot came before this barrier
#pragma unroll
    for (int tb = 0; tb < TB; tb++)
#pragma unroll
      for (int cb = 0; cb < CB; cb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          float v;
          ot[16 * tb + 4 * kg + i][col0 + 16 * cb + n] =
              (unsigned short)round16<DT>(acc[tb][cb][i] * (1.f / Split<DT>::kScale), &v);
        }
    __syncthreads();

#pragma unroll
    for (int u = 0; u < CPT; u++) {
      const int c = tid + u * NT, tt = c / 16, j0 = (c % 16) * 8, t = t0 + tt;
      if (t < t_end) {
        const size_t row = (size_t)(p.pos + t);
        const size_t e0 = j0 < sh.dp ? row * sh.dp + j0
                                     : sh.kl.rest_off + row * sh.kl.rest + (j0 - sh.dp);
        __builtin_nontemporal_store(
            *reinterpret_cast<const u32x4*>(&ot[tt][j0]),
            reinterpret_cast<u32x4*>(static_cast<unsigned short*>(p.kcache) +
                                     head * sh.kl.head_elems + e0));
      }
    }
  };

  for (int t0 = t_begin; t0 < t_end; t0 += DEPTH * kPreTile) {
#pragma unroll
    for (int b = 0; b < DEPTH; b++)
      if (t0 + b * kPreTile < t_end) tile(xk[b], t0 + b * kPreTile);
  }
}

// Thread (slot, j) keeps column j of P[kv] in registers and forms coordinate j
// of tokens slot, slot + NSLOT, ... of each run of RUN tokens staged in LDS;
// a workgroup covers tpwg tokens.
template <int DT, int D>
__global__ __launch_bounds__(kPreThreads) void prefill_valu_kernel(PrefillParams p, int tpwg) {
  constexpr int NSLOT = kPreThreads / D, RUN = 32;
  __shared__ __align__(16) float xs[RUN][D];
  const Shape& sh = p.sh;
  const size_t head = blockIdx.y;
  const int kv = (int)(head % sh.Hkv);
  // (D = 96: the threads past NSLOT*D only help stage the keys)
  const int j = threadIdx.x % D, slot = threadIdx.x / D;
  const bool has_col = slot < NSLOT;
  float pc[D];
  {
    const float* P = p.P + (size_t)kv * D * D;
#pragma unroll
    for (int i = 0; i < D; i++) pc[i] = P[(size_t)i * D + j];
  }
  const int t_begin = blockIdx.x * tpwg;
  const int t_end = min(p.n_tokens, t_begin + tpwg);
  for (int t0 = t_begin; t0 < t_end; t0 += RUN) {
    __syncthreads();  // previous run consumed
    for (int e = threadIdx.x; e < RUN * D; e += kPreThreads) {
      const int t = t0 + e / D;
      xs[e / D][e % D] = t < t_end ? load_elem<DT>(p.k_rows, (head * p.n_tokens + t) * D + e % D) : 0.f;
    }
    __syncthreads();
#pragma unroll 1
    for (int r = slot; has_col && r < RUN && t0 + r < t_end; r += NSLOT) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < D; i += 4) {
        const float4 x = *reinterpret_cast<const float4*>(&xs[r][i]);
        a = fmaf(x.x, pc[i], a);
        a = fmaf(x.y, pc[i + 1], a);
        a = fmaf(x.z, pc[i + 2], a);
        a = fmaf(x.w, pc[i + 3], a);
      }
      store_elem<DT>(p.kcache, sh.kl.at(head, (size_t)(p.pos + t0 + r), j), a);
    }
  }
}

// Tokens per workgroup from a list of candidates: the largest whose whole
// rounds of resident workgroups (a last partial round costs as much as a full
// one) take least time, each workgroup costing its tokens plus `setup` tokens'
// worth (loading its part of P).
static int pick_tokens(const PrefillParams& p, int per_cu, const int* cand, int n_cand, int setup) {
  const long long slots = (long long)per_cu * (p.cus > 0 ? p.cus : 256);
  const long long heads = (long long)p.sh.B * p.sh.Hkv;
  int best = 0;
  long long best_cost = 0;
  for (int i = 0; i < n_cand; i++) {
    const int t = cand[i];
    const long long wgs = (p.n_tokens + t - 1) / t * heads;
    const long long cost = (wgs + slots - 1) / slots * (t + setup);
    if (best == 0 || cost < best_cost) best = t, best_cost = cost;
  }
  return best;
}

template <int DT, int TPWG>
hipError_t launch_mfma(const PrefillParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((p.n_tokens + TPWG - 1) / TPWG), (unsigned)(p.sh.B * p.sh.Hkv));
  prefill_mfma_kernel<DT, kPreWaves, kPreDepth, TPWG><<<grid, 64 * kPreWaves, 0, st>>>(p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_mfma_sized(const PrefillParams& p, hipStream_t st) {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nb, prefill_mfma_kernel<DT, kPreWaves, kPreDepth, 1024>, 64 * kPreWaves, 0) !=
            hipSuccess || nb < 1)
      nb = 1;
    return nb;
  }();
  static const int cand[] = {4096, 2048, 1024, 512};
  switch (pick_tokens(p, per_cu, cand, 4, 128)) {
    case 4096: return launch_mfma<DT, 4096>(p, st);
    case 2048: return launch_mfma<DT, 2048>(p, st);
    case 1024: return launch_mfma<DT, 1024>(p, st);
    default: return launch_mfma<DT, 512>(p, st);
  }
}

template <int DT, int D>
hipError_t launch_valu(const PrefillParams& p, hipStream_t st) {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, prefill_valu_kernel<DT, D>, kPreThreads,
                                                     0) != hipSuccess || nb < 1)
      nb = 1;
    return nb;
  }();
  static const int cand[] = {512, 256, 128, 64};
  const int tpwg = pick_tokens(p, per_cu, cand, 4, 32);
  const dim3 grid((unsigned)((p.n_tokens + tpwg - 1) / tpwg), (unsigned)(p.sh.B * p.sh.Hkv));
  prefill_valu_kernel<DT, D><<<grid, kPreThreads, 0, st>>>(p, tpwg);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const PrefillParams& p, hipStream_t st) {
  if constexpr (DT != F32) {
    if (p.sh.D == 128) return launch_mfma_sized<DT>(p, st);
  }
  switch (p.sh.D) {
    case 128: return launch_valu<DT, 128>(p, st);
    case 96: return launch_valu<DT, 96>(p, st);
    default: return launch_valu<DT, 64>(p, st);
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t st) {
  switch (p.sh.dtype) {
    case F32: return launch_dt<F32>(p, st);
    case F16: return launch_dt<F16>(p, st);
    default: return launch_dt<BF16>(p, st);
  }
}

}  // namespace loki
