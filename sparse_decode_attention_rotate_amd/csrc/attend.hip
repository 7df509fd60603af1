// Exact softmax attention over the selected tokens only, split-k.
//
// Loki (poster page, "TL;DR"; "Visual Insights", Figure 1 right): the
// full-dimensional keys of the k selected tokens give the final attention
// scores; softmax and the value sum run over those k tokens.
//
// Workgroup (split, b*Hq+h) stages up to p.kc of the selected token
// indices in LDS and runs block_attend (attend_core.h) over them.  With one
// split it writes the output row; otherwise it writes (m, l, acc[D]) in the
// log2 domain and combine_kernel merges the splits.
//
// Without an index list (idx == null) row r is token r: dense decode
// attention over all S cached tokens, the full-attention baseline the pages
// compare Loki with (poster page "TL;DR": speed-up over vanilla attention).
// With low_dim set as well the logits use only the leading d rotated
// coordinates: PCAAttn, the Loki variant that attends with the
// reduced-dimensional scores directly (poster page, "More on tables").
#include "attend_core.h"
#include "loki_internal.h"

namespace loki {

namespace {

constexpr int kAttThreads = 256;
constexpr int kXcds = 8;  // MI355X: workgroup i runs on XCD i % 8

template <int DT, int D, bool SPLIT, bool LOW, bool STREAM>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttendParams p) {
  // the chunk's index list and partial logits: p.kc entries each (dynamic
  // LDS sized by the launch, so that small chunks keep small workgroups)
  extern __shared__ __align__(16) unsigned char att_lists[];
  int* sidx = reinterpret_cast<int*>(att_lists);
  float* slow = reinterpret_cast<float*>(att_lists + (size_t)p.kc * 4);
  __shared__ AttendSmem<DT, D, kAttThreads> sm;

  const Shape& sh = p.sh;
  // Grouped heads gathering selected rows: workgroups are dealt to the 8 XCDs
  // round-robin by index, so the g * nsplit workgroups of one (b, kv) group
  // are given indices that fall on the same XCD, where the rows the heads
  // share meet in one L2.  (Without index lists -- every token -- the plain
  // order already puts the g heads of one chunk on one XCD at the same time.)
  int wg = (int)blockIdx.x;
  if (sh.g > 1 && p.idx) {
    const int per = sh.g * p.nsplit;
    const int x = wg % kXcds, s = wg / kXcds;
    wg = ((s / per) * kXcds + x) * per + s % per;
    if (wg >= p.nsplit * sh.B * sh.Hq) return;  // padding of the last groups
  }
  const int split = wg % p.nsplit;
  const size_t bh = (size_t)(wg / p.nsplit);
  const int b = (int)(bh / sh.Hq), h = (int)(bh % sh.Hq);
  const size_t head = (size_t)b * sh.Hkv + h / sh.g;
  const int r0 = split * p.kc;
  const int nr = min(p.kc, p.k - r0);
  const int tid = threadIdx.x;

  // the chunk's token indices (invalid ones as -1) and low-dim partial logits
  for (int r = tid; r < nr; r += kAttThreads) {
    const int t = p.idx ? p.idx[bh * p.k + r0 + r] : r0 + r;
    sidx[r] = (t >= 0 && t < sh.S) ? t : -1;
    if (SPLIT) slow[r] = p.sel_scores[bh * p.k + r0 + r];
  }
  __syncthreads();

  float M, L, A;
  block_attend<DT, D, kAttThreads, SPLIT, kRowsPerBatch, LOW, STREAM>(
      p.qr + bh * D, p.scale_log2, sidx, slow, nr, p.kcache, p.vcache, head, sh, sm, M, L, A, p.d);
  if (tid < D) {
    if (p.nsplit == 1) {
      store_out(p.out, bh * D + tid, A / L, sh.odt);
    } else {
      float* part = p.part + (bh * p.nsplit + split) * (size_t)(D + 2);
      part[2 + tid] = A;
      if (tid == 0) {
        part[0] = M;
        part[1] = L;
      }
    }
  }
}

// Merges the splits of one row: M = max of the splits' maxima, each split
// weighted by 2^(m_s - M), added in split order.  The kernel is all latency
// (a few hundred KB of partials, written by other XCDs, so not in this
// XCD's L2): the first block's (m, l) and the first batch of accumulators
// are loaded together, and each later batch of kBatch splits is one round
// trip instead of one per split.
template <int D>
__global__ __launch_bounds__(kLaneDim<D>) void combine_kernel(AttendParams p) {
  // NTH threads (D, or 128 for D = 96): thread t loads the (m, l) of splits
  // t, t + NTH, ... and, when t < D, forms output coordinate t
  constexpr int NTH = kLaneDim<D>;
  constexpr int kBatch = 8;
  constexpr int kWaves = NTH / 64;
  __shared__ float sw[NTH], sl[NTH], smax[kWaves];
  const int tid = threadIdx.x, ns = p.nsplit;
  const int col = tid < D ? tid : 0;  // threads past D read column 0 and store nothing
  const size_t bh = blockIdx.x;
  const size_t stride = D + 2;
  const float* part = p.part + bh * ns * stride;

  float mo = -INFINITY, lo = 0.f;
  if (tid < ns) {
    mo = part[tid * stride];
    lo = part[tid * stride + 1];
  }
  float v[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; j++) v[j] = j < ns ? part[j * stride + 2 + col] : 0.f;
  float m = mo;
  for (int s = tid + NTH; s < ns; s += NTH) m = fmaxf(m, part[s * stride]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) smax[tid >> 6] = m;
  __syncthreads();
  float M = smax[0];
#pragma unroll
  for (int w = 1; w < kWaves; w++) M = fmaxf(M, smax[w]);

  float L = 0.f, a = 0.f;
  for (int b0 = 0; b0 < ns; b0 += NTH) {
    if (b0 > 0) {
      __syncthreads();  // every thread is done with the previous block's weights
      mo = -INFINITY;
      lo = 0.f;
      if (b0 + tid < ns) {
        mo = part[(b0 + tid) * stride];
        lo = part[(b0 + tid) * stride + 1];
      }
    }
    sw[tid] = mo == -INFINITY ? 0.f : exp2f(mo - M);
    sl[tid] = lo;
    __syncthreads();
    const int nb = min(NTH, ns - b0);
    for (int j0 = 0; j0 < nb; j0 += kBatch) {
      if (b0 + j0 > 0) {  // the first batch was loaded up front
#pragma unroll
        for (int j = 0; j < kBatch; j++)
          v[j] = j0 + j < nb ? part[(b0 + j0 + j) * stride + 2 + col] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kBatch; j++) {
        if (j0 + j < nb) {
          L = fmaf(sl[j0 + j], sw[j0 + j], L);
          a = fmaf(v[j], sw[j0 + j], a);
        }
      }
    }
  }
  if (tid < D) store_out(p.out, bh * D + tid, a / L, p.sh.odt);
}

template <int DT, int D>
hipError_t launch_d(const AttendParams& p, hipStream_t st) {
  // grouped heads with index lists: whole groups of kXcds (b, kv) units, so
  // that each XCD gets the workgroups of its groups (the padding workgroups
  // return at once)
  const size_t groups = (size_t)p.sh.B * p.sh.Hkv;
  const dim3 grid((unsigned)(p.sh.g == 1 || !p.idx
                                 ? (size_t)p.nsplit * p.sh.B * p.sh.Hq
                                 : (groups + kXcds - 1) / kXcds * kXcds * p.sh.g * p.nsplit));
  // Load policy: index lists are streamed (nontemporal) -- grouped heads
  // select mostly different rows (their sets overlap by ~15-20% here), so the
  // stream rate is worth more than the reuse; every token with grouped heads
  // keeps the default policy, so that the g heads reading each chunk share it
  // in L2.
  const bool once = p.sh.g == 1 || p.idx != nullptr;
  const size_t lists = (size_t)p.kc * 8;  // sidx + slow
  if (p.sel_scores) {
    if (once)
      attend_kernel<DT, D, true, false, true><<<grid, kAttThreads, lists, st>>>(p);
    else
      attend_kernel<DT, D, true, false, false><<<grid, kAttThreads, lists, st>>>(p);
  } else if (p.low_dim) {
    if (once)
      attend_kernel<DT, D, false, true, true><<<grid, kAttThreads, lists, st>>>(p);
    else
      attend_kernel<DT, D, false, true, false><<<grid, kAttThreads, lists, st>>>(p);
  } else {
    if (once)
      attend_kernel<DT, D, false, false, true><<<grid, kAttThreads, lists, st>>>(p);
    else
      attend_kernel<DT, D, false, false, false><<<grid, kAttThreads, lists, st>>>(p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  combine_kernel<D><<<dim3((unsigned)(p.sh.B * p.sh.Hq)), kLaneDim<D>, 0, st>>>(p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const AttendParams& p, hipStream_t st) {
  switch (p.sh.D) {
    case 128: return launch_d<DT, 128>(p, st);
    case 96: return launch_d<DT, 96>(p, st);
    default: return launch_d<DT, 64>(p, st);
  }
}

}  // namespace

hipError_t launch_attend(const AttendParams& p, hipStream_t st) {
  switch (p.sh.dtype) {
    case F32: return launch_dt<F32>(p, st);
    case F16: return launch_dt<F16>(p, st);
    default: return launch_dt<BF16>(p, st);
  }
}

}  // namespace loki
