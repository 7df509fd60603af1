// Device-side helpers shared by the Loki kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace loki {

enum Dtype : int { F32 = 0, F16 = 1, BF16 = 2 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int DT> struct Elem;
template <> struct Elem<F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;  // elements in one 16-byte load
};
template <> struct Elem<F16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
};
template <> struct Elem<BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
};

// ---------------------------------------------------------------- dtype I/O

// One 16-byte vector -> kPerVec floats (exact widening).
template <int DT> __device__ __forceinline__ void unpack16(u32x4 v, float* f);

template <> __device__ __forceinline__ void unpack16<F32>(u32x4 v, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

template <> __device__ __forceinline__ void unpack16<F16>(u32x4 v, float* f) {
  f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
  for (int i = 0; i < 8; i++) f[i] = (float)h[i];
}

template <> __device__ __forceinline__ void unpack16<BF16>(u32x4 v, float* f) {
  // element 2w sits in the low half of dword w (little endian)
  unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <int DT> __device__ __forceinline__ float load_elem(const void* base, size_t i);
template <> __device__ __forceinline__ float load_elem<F32>(const void* base, size_t i) {
  return static_cast<const float*>(base)[i];
}
template <> __device__ __forceinline__ float load_elem<F16>(const void* base, size_t i) {
  return (float)static_cast<const _Float16*>(base)[i];
}
template <> __device__ __forceinline__ float load_elem<BF16>(const void* base, size_t i) {
  return __uint_as_float((unsigned)static_cast<const unsigned short*>(base)[i] << 16);
}

// fp32 -> storage dtype, round to nearest, ties to even.
template <int DT> __device__ __forceinline__ void store_elem(void* base, size_t i, float x);
template <> __device__ __forceinline__ void store_elem<F32>(void* base, size_t i, float x) {
  static_cast<float*>(base)[i] = x;
}
template <> __device__ __forceinline__ void store_elem<F16>(void* base, size_t i, float x) {
  static_cast<_Float16*>(base)[i] = (_Float16)x;
}
__device__ __forceinline__ unsigned short bf16_bits(float x) {
  unsigned u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);  // round half to even on bit 16
  return (unsigned short)(u >> 16);
}
template <> __device__ __forceinline__ void store_elem<BF16>(void* base, size_t i, float x) {
  static_cast<unsigned short*>(base)[i] = bf16_bits(x);
}

// An attention output element in the output dtype (uniform across the wave).
__device__ __forceinline__ void store_out(void* base, size_t i, float x, int odt) {
  if (odt == F32)
    store_elem<F32>(base, i, x);
  else if (odt == F16)
    store_elem<F16>(base, i, x);
  else
    store_elem<BF16>(base, i, x);
}

// The value store_elem<DT> keeps, as fp32.
template <int DT> __device__ __forceinline__ float stored_value(float x);
template <> __device__ __forceinline__ float stored_value<F32>(float x) { return x; }
template <> __device__ __forceinline__ float stored_value<F16>(float x) {
  return (float)(_Float16)x;
}
template <> __device__ __forceinline__ float stored_value<BF16>(float x) {
  return __uint_as_float((unsigned)bf16_bits(x) << 16);
}

// Raw element copy (no conversion), for moving stored rows.
template <int DT> __device__ __forceinline__ void copy_elem(void* dst, size_t di, const void* src,
                                                            size_t si) {
  if constexpr (Elem<DT>::kBytes == 4)
    static_cast<unsigned*>(dst)[di] = static_cast<const unsigned*>(src)[si];
  else
    static_cast<unsigned short*>(dst)[di] = static_cast<const unsigned short*>(src)[si];
}

// ---------------------------------------------------------------- buffer loads
//
// Raw buffer loads carry a hardware range check: a load whose byte offset lies
// past the descriptor's size returns zeros and touches no memory.  Loads of
// rows that do not exist (tails, invalid indices) therefore need no branch,
// which keeps every load of a batch in flight together.

typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  // word 3 of a gfx9 buffer descriptor: 32-bit data format, no swizzle
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 load16(Rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}
// Same, with the nontemporal cache policy: for data read once (cache
// streams); on MI355X a read stream with it runs at ~7.0 TB/s against
// ~6.2 TB/s with the default policy.
__device__ __forceinline__ u32x4 load16_stream(Rsrc r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2));
}

// ---------------------------------------------------------------- cross-lane

// DPP move within a row of 16 lanes (ctrl is the gfx9 DPP control word).
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of L lanes; every lane of a group gets the group sum.
template <int L> __device__ __forceinline__ float group_sum(float v) {
  if constexpr (L >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (L >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (L >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
  if constexpr (L >= 16) v += dpp_f<0x140>(v);  // row_mirror
  if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// DPP shift within a row with zero fill for lanes that have no source.
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ unsigned dpp_shift_u(unsigned x) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWMASK, 0xf, false);
}

// Inclusive prefix sum across the 64 lanes of a wave, DPP only.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned x) {
  x += dpp_shift_u<0x111>(x);          // row_shr:1
  x += dpp_shift_u<0x112>(x);          // row_shr:2
  x += dpp_shift_u<0x114>(x);          // row_shr:4
  x += dpp_shift_u<0x118>(x);          // row_shr:8   (prefix within each row of 16)
  x += dpp_shift_u<0x142, 0xa>(x);     // row_bcast:15 into rows 1 and 3
  x += dpp_shift_u<0x143, 0xc>(x);     // row_bcast:31 into rows 2 and 3
  return x;
}

// Number of set bits of a wave ballot below this lane.
__device__ __forceinline__ int lane_rank(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
}

// ---------------------------------------------------------------- paired workgroups
//
// Words exchanged between the two workgroups of a paired unit are accessed
// only with agent-coherent loads and stores (relaxed agent-scope atomics,
// which bypass the non-coherent caches): a workgroup waits until its stores
// are complete before it touches the pair's flag, and reads its partner's
// words only after the flag showed the partner had been there.  No cache
// writeback or invalidate is needed (release / acquire fences would write
// back or invalidate a whole L2 each time, at a cost to every workgroup on
// that die).
__device__ __forceinline__ void st_coherent(float* a, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(a), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* a) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned*>(a), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
// cache policy of a buffer access with the agent-coherent bit (sc1), as the
// agent-scope accesses above: for 16-byte loads of words stored that way
constexpr int kCoherentSc1 = 16;

// ---------------------------------------------------------------- K cache layout
//
// Split-panel rotated key cache.  Per (batch, KV head) one block of S_cap*D
// elements: first the leading `dp` rotated coordinates of every token
// (token-major, S_cap x dp), then the remaining D-dp coordinates
// (S_cap x (D-dp)).  Scoring streams the first part contiguously; the final
// attention reads the second part of the selected rows.
struct KLayout {
  size_t head_elems;  // S_cap * D
  size_t rest_off;    // S_cap * dp
  int dp;             // panel width
  int rest;           // D - dp

  __host__ __device__ size_t at(size_t head, size_t t, int j) const {
    return head * head_elems +
           (j < dp ? t * (size_t)dp + j : rest_off + t * (size_t)rest + (size_t)(j - dp));
  }
};

}  // namespace loki
