// Phase timestamps of the one-launch kernels, for profiling builds only.
//
// Built with LOKI_PHASE_STAMPS defined (the library libloki_stamps.so, built
// by `python -m sparse_decode_attention_rotate_amd.build --stamps`), thread 0
// of each workgroup records the constant 100 MHz clock (s_memrealtime) at the
// boundaries of its phases into a per-kernel device array, and the last slot holds
// the workgroup's HW_ID register (compute unit, shader engine); the library
// exports loki_phase_stamps_fused / loki_phase_stamps_head to copy them out.
// In the product library every stamp compiles to nothing.
#pragma once

#include <hip/hip_runtime.h>

namespace loki {
constexpr int kStampSlots = 16;           // per workgroup: phase boundaries 0..14, HW_ID at 15
constexpr int kStampWorkgroups = 8192;    // workgroups recorded (the first ones of a launch)
}  // namespace loki

#ifdef LOKI_PHASE_STAMPS
#define LOKI_STAMP_ARRAY(name) \
  static __device__ unsigned long long name[loki::kStampWorkgroups * loki::kStampSlots]
#define LOKI_STAMP(arr, i)                                                             \
  do {                                                                                 \
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)loki::kStampWorkgroups)             \
      arr[blockIdx.x * loki::kStampSlots + (i)] = __builtin_amdgcn_s_memrealtime();    \
  } while (0)
// HW_ID (hwreg 4, all 32 bits)
#define LOKI_STAMP_HWID(arr)                                                           \
  do {                                                                                 \
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)loki::kStampWorkgroups)             \
      arr[blockIdx.x * loki::kStampSlots + loki::kStampSlots - 1] =                                        \
          (unsigned)__builtin_amdgcn_s_getreg((31 << 11) | 4);                         \
  } while (0)
#define LOKI_STAMP_EXPORT(fn, arr)                                                     \
  extern "C" int fn(void* host, size_t n_workgroups) {                                 \
    if (n_workgroups > (size_t)loki::kStampWorkgroups) n_workgroups = loki::kStampWorkgroups; \
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(arr),                             \
                                    n_workgroups * loki::kStampSlots * 8, 0,           \
                                    hipMemcpyDeviceToHost);                            \
  }
#else
#define LOKI_STAMP_ARRAY(name) static_assert(true, "")
#define LOKI_STAMP(arr, i) \
  do {                     \
  } while (0)
#define LOKI_STAMP_HWID(arr) \
  do {                       \
  } while (0)
#define LOKI_STAMP_EXPORT(fn, arr) static_assert(true, "")
#endif
