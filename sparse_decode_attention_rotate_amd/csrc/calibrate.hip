// Calibration of the rotation P on the GPU: principal component analysis of
// a set of calibration keys per KV head (poster page, "Visual Insights",
// Figure 1 right, and "More on figures": PCA of keys from a calibration set,
// done offline, gives the basis the keys and queries are rotated into).
//
// Covariance.  C = (1/n) sum_t (x_t - mu)(x_t - mu)^T.  The keys are shifted
// by the head's first calibration key c, so that a large common mean cannot
// cancel digits: with y_t = x_t - c, C = S2/n - m m^T, S2 = sum_t y_t y_t^T,
// m = (1/n) sum_t y_t.  S2 is a dense [D x n] . [n x D] product: MFMA
// 16x16x32 bf16, y split into three bf16 parts (y1 + y2 + y3 = y exactly for
// normal fp32 values), the part products of weight above 2^-24 kept
// (1.1, 1.2, 2.1, 2.2, 1.3, 3.1) and accumulated in fp32.  Workgroup
// (chunk, kv) sums kCalChunk tokens; its partial sums go to the workspace.
//
// Eigenvectors.  One workgroup per KV head sums the partials in chunk order,
// then runs the cyclic Jacobi method on A = C (fp32, LDS) with the
// round-robin ordering: D/2 disjoint rotations per step, D-1 steps per sweep,
// each rotation chosen to zero its off-diagonal pair (the symmetric 2 x 2
// Schur decomposition of Golub & Van Loan), the rotations accumulated in V.
// It stops after a sweep that needs no rotation (every off-diagonal entry
// below 2^-23 sqrt(|a_pp a_qq|)) or after kJacMaxSweeps.  The columns of V are
// then normalised, ordered by descending eigenvalue (equal ones by index),
// signed so that their first largest-magnitude entry is positive, and written
// as the columns of P; the eigenvalues are the variances.
#include "loki_internal.h"

namespace loki {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kCalTile = 64;        // tokens per LDS stage
constexpr int kJacThreads = 1024;
constexpr int kJacMaxSweeps = 40;

// x rounded to nearest-even bf16: bits; *back = its value (finite x)
__device__ __forceinline__ unsigned short bf16_part(float x, float* back) {
  unsigned u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  const unsigned short b = (unsigned short)(u >> 16);
  *back = __uint_as_float((unsigned)b << 16);
  return b;
}

__device__ __forceinline__ float4_t mfma_bf16(u32x4 a, u32x4 b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Operand layout of the 16x16x32 product: lane l supplies row l%16 of A and
// column l%16 of B at the inner indices 8*(l/16) .. +7; result element i of
// lane l is row 4*(l/16)+i, column l%16.  Here both operands are slices of
// the transposed tile yt[part][dimension][token]: A = yT rows (16w ..), B =
// y columns (16cb ..), inner index = token.
template <int DT, int D>
__global__ __launch_bounds__(4 * D) void calib_cov_kernel(CalibParams p) {
  constexpr int NT = 4 * D, NW = D / 16, TPP = NT / D;  // TPP: tokens staged per pass
  constexpr int RP = kCalTile + 8;                      // padded token row (bf16 elements)
  __shared__ __align__(16) unsigned short yt[3][D][RP];
  __shared__ float shift[D];
  __shared__ float s1red[TPP][D];

  const int kv = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane % 16, kg = lane / 16;
  const size_t kbase = (size_t)kv * p.n * D;
  const int t_begin = chunk * kCalChunk, t_end = min(p.n, t_begin + kCalChunk);
  if (tid < D) shift[tid] = load_elem<DT>(p.keys, kbase + tid);
  __syncthreads();
  const int dim = tid % D, trow = tid / D;
  const float c = shift[dim];
  float s1 = 0.f;
  float4_t acc[NW];
#pragma unroll
  for (int cb = 0; cb < NW; cb++) acc[cb] = float4_t{0.f, 0.f, 0.f, 0.f};

  for (int t0 = t_begin; t0 < t_end; t0 += kCalTile) {
    // stage y = x - c, split in three bf16 parts, dimension-major
#pragma unroll 4
    for (int r = trow; r < kCalTile; r += TPP) {
      const int t = t0 + r;
      float y = t < t_end ? load_elem<DT>(p.keys, kbase + (size_t)t * D + dim) - c : 0.f;
      s1 += y;
      float v;
      yt[0][dim][r] = bf16_part(y, &v);
      y -= v;
      yt[1][dim][r] = bf16_part(y, &v);
      y -= v;
      yt[2][dim][r] = bf16_part(y, &v);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kCalTile / 32; ks++) {
      const int col = 32 * ks + 8 * kg;
      u32x4 a[3];
#pragma unroll
      for (int s = 0; s < 3; s++) a[s] = *reinterpret_cast<const u32x4*>(&yt[s][16 * wave + n][col]);
#pragma unroll
      for (int cb = 0; cb < NW; cb++) {
        u32x4 b[3];
#pragma unroll
        for (int s = 0; s < 3; s++) b[s] = *reinterpret_cast<const u32x4*>(&yt[s][16 * cb + n][col]);
        acc[cb] = mfma_bf16(a[0], b[0], acc[cb]);
        acc[cb] = mfma_bf16(a[0], b[1], acc[cb]);
        acc[cb] = mfma_bf16(a[1], b[0], acc[cb]);
        acc[cb] = mfma_bf16(a[1], b[1], acc[cb]);
        acc[cb] = mfma_bf16(a[0], b[2], acc[cb]);
        acc[cb] = mfma_bf16(a[2], b[0], acc[cb]);
      }
    }
    __syncthreads();  // yt is rewritten by the next stage
  }

  float* s2 = p.part_s2 + ((size_t)kv * p.nch + chunk) * D * D;
#pragma unroll
  for (int cb = 0; cb < NW; cb++)
#pragma unroll
    for (int i = 0; i < 4; i++) s2[(size_t)(16 * wave + 4 * kg + i) * D + 16 * cb + n] = acc[cb][i];
  s1red[trow][dim] = s1;
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < TPP; r++) s += s1red[r][tid];
    p.part_s1[((size_t)kv * p.nch + chunk) * D + tid] = s;
  }
}

template <int D>
__global__ __launch_bounds__(kJacThreads) void calib_eigen_kernel(CalibParams p) {
  constexpr int HP = D / 2, RP = D + 1;
  __shared__ float A[D][RP];
  __shared__ float V[D][RP];
  __shared__ float m[D];
  __shared__ int pp[HP], qq[HP], rf[HP];
  __shared__ float cc[HP], ss[HP], dpp[HP], dqq[HP];
  __shared__ float lam[D], colscale[D];
  __shared__ int rank[D];
  __shared__ int n_rot;
  __shared__ float floor_abs;

  const int kv = blockIdx.x, tid = threadIdx.x;
  const float inv_n = 1.f / (float)p.n;
  if (tid < D) {
    float s = 0.f;
    for (int ch = 0; ch < p.nch; ch++) s += p.part_s1[((size_t)kv * p.nch + ch) * D + tid];
    m[tid] = s * inv_n;
  }
  __syncthreads();
  for (int e = tid; e < D * D; e += kJacThreads) {
    const int i = e / D, j = e % D;
    float s = 0.f;
    for (int ch = 0; ch < p.nch; ch++)
      s += p.part_s2[(((size_t)kv * p.nch + ch) * D + i) * D + j];
    A[i][j] = s * inv_n - m[i] * m[j];
    V[i][j] = i == j ? 1.f : 0.f;
  }
  __syncthreads();
  // symmetrise (the two triangles were summed in different orders)
  for (int e = tid; e < D * D; e += kJacThreads) {
    const int i = e / D, j = e % D;
    if (i < j) {
      const float a = 0.5f * (A[i][j] + A[j][i]);
      A[i][j] = a;
      A[j][i] = a;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float tr = 0.f;
    for (int i = 0; i < D; i++) tr += fabsf(A[i][i]);
    floor_abs = tr * 0x1p-46f;  // off-diagonal entries below this are taken as zero
  }

  for (int sweep = 0; sweep < kJacMaxSweeps; sweep++) {
    if (tid == 0) n_rot = 0;
    __syncthreads();
    for (int r = 0; r < D - 1; r++) {
      if (tid < HP) {
        const int k = tid;
        const int p_ = k == 0 ? 0 : 1 + (k - 1 + r) % (D - 1);
        const int q_ = 1 + (D - 2 - k + r) % (D - 1);
        const float apq = A[p_][q_], app = A[p_][p_], aqq = A[q_][q_];
        float c = 1.f, s = 0.f, t = 0.f;
        const bool rot = fabsf(apq) > fmaxf(0x1p-23f * sqrtf(fabsf(app * aqq)), floor_abs);
        if (rot) {
          const float tau = (aqq - app) / (2.f * apq);
          t = (tau >= 0.f ? 1.f : -1.f) / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + t * t);
          s = t * c;
          atomicAdd(&n_rot, 1);
        }
        pp[k] = p_;
        qq[k] = q_;
        cc[k] = c;
        ss[k] = s;
        dpp[k] = app - t * apq;
        dqq[k] = aqq + t * apq;
        rf[k] = rot;
      }
      __syncthreads();
      // rows p, q of every rotated pair: A <- J^T A
      for (int e = tid; e < HP * D; e += kJacThreads) {
        const int k = e / D, j = e % D;
        if (!rf[k]) continue;
        const int p_ = pp[k], q_ = qq[k];
        const float c = cc[k], s = ss[k];
        const float x = A[p_][j], y = A[q_][j];
        A[p_][j] = c * x - s * y;
        A[q_][j] = s * x + c * y;
      }
      __syncthreads();
      // columns p, q: A <- A J (the pair's own 2 x 2 block set exactly), V <- V J
      for (int e = tid; e < HP * D; e += kJacThreads) {
        const int k = e / D, i = e % D;
        if (!rf[k]) continue;
        const int p_ = pp[k], q_ = qq[k];
        const float c = cc[k], s = ss[k];
        if (i != p_ && i != q_) {
          const float x = A[i][p_], y = A[i][q_];
          A[i][p_] = c * x - s * y;
          A[i][q_] = s * x + c * y;
        } else if (i == p_) {
          A[p_][p_] = dpp[k];
          A[q_][q_] = dqq[k];
          A[p_][q_] = 0.f;
          A[q_][p_] = 0.f;
        }
        const float vx = V[i][p_], vy = V[i][q_];
        V[i][p_] = c * vx - s * vy;
        V[i][q_] = s * vx + c * vy;
      }
      __syncthreads();
    }
    const bool done = n_rot == 0;
    __syncthreads();  // every thread has read n_rot before it is reset
    if (done) break;
  }

  // eigenvalue order, column norms and signs
  if (tid < D) {
    const int i = tid;
    const float li = A[i][i];
    float nrm = 0.f, best = -1.f;
    int arg = 0;
    for (int r = 0; r < D; r++) {
      const float v = V[r][i];
      nrm = fmaf(v, v, nrm);
      if (fabsf(v) > best) {
        best = fabsf(v);
        arg = r;
      }
    }
    int rk = 0;
    for (int j = 0; j < D; j++) {
      const float lj = A[j][j];
      rk += (lj > li) || (lj == li && j < i);
    }
    lam[i] = li;
    rank[i] = rk;
    colscale[i] = (V[arg][i] < 0.f ? -1.f : 1.f) / sqrtf(nrm);
  }
  __syncthreads();
  float* P = p.P + (size_t)kv * D * D;
  for (int e = tid; e < D * D; e += kJacThreads) {
    const int r = e / D, i = e % D;
    P[(size_t)r * D + rank[i]] = V[r][i] * colscale[i];
  }
  if (p.variances && tid < D) p.variances[(size_t)kv * D + rank[tid]] = lam[tid];
}

template <int DT, int D>
hipError_t launch_d(const CalibParams& p, hipStream_t st) {
  calib_cov_kernel<DT, D><<<dim3((unsigned)p.nch, (unsigned)p.sh.Hkv), 4 * D, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  calib_eigen_kernel<D><<<dim3((unsigned)p.sh.Hkv), kJacThreads, 0, st>>>(p);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const CalibParams& p, hipStream_t st) {
  switch (p.sh.D) {
    case 128: return launch_d<DT, 128>(p, st);
    case 96: return launch_d<DT, 96>(p, st);
    default: return launch_d<DT, 64>(p, st);
  }
}

}  // namespace

hipError_t launch_calibrate(const CalibParams& p, hipStream_t st) {
  switch (p.sh.dtype) {
    case F32: return launch_dt<F32>(p, st);
    case F16: return launch_dt<F16>(p, st);
    default: return launch_dt<BF16>(p, st);
  }
}

}  // namespace loki
