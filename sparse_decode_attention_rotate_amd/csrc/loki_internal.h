// Kernel parameter blocks and launcher declarations (library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "loki_common.h"

namespace loki {

struct Shape {
  int B, Hq, Hkv, g, D, S, S_cap, dp, dtype;
  int odt;  // dtype of the attention output
  KLayout kl;
};

struct ProjectParams {
  const void* q;      // [B,Hq,D] storage dtype (nullable: no query rotation)
  const void* k_new;  // [B,Hkv,D] (nullable: no append)
  const void* v_new;  // [B,Hkv,D]
  const float* P;     // [Hkv,D,D]
  float* qr;          // [B,Hq,D] fp32
  void* kcache;
  void* vcache;
  int pos;            // append row
  int bb;             // batch rows per workgroup
  hipStream_t stream;
  Shape sh;
};

struct ScoreParams {
  const float* qr;     // [B,Hq,D]
  const void* q;       // [B,Hq,D] storage dtype, nullable: rotate q by P in the kernel
  const float* P;      // [Hkv,D,D] (with q)
  float* qr_out;       // [B,Hq,D] the rotated rows, written by each unit's first tile (with q)
  const void* k_new;   // [B,Hkv,D] nullable (with q): appended as token S-1 by each unit's last tile
  const void* v_new;   // [B,Hkv,D]
  void* kcache_w;      // the caches, written at row S-1 when appending
  void* vcache_w;
  const void* kcache;
  float* scores;       // [B,Hq,S]
  int d;
  int n_tiles;         // tiles per (b, kv)
  int tile_tokens;     // tokens per tile (panel kernel)
  Shape sh;
};

struct TopkParams {
  const float* scores;  // [B*Hq, S]
  int32_t* idx;         // [B*Hq, k] ascending
  float* sel_scores;    // [B*Hq, k] nullable: low-dim score of each selected token
  int S, k;
};

struct AttendParams {
  const float* qr;          // [B,Hq,D]
  const void* kcache;
  const void* vcache;
  const int32_t* idx;       // [B*Hq, k]; null: row r is token r (k = S, dense attention)
  const float* sel_scores;  // [B*Hq, k] low-dim partial logits (split variant) or null
  void* out;                // [B,Hq,D] in sh.odt (written when nsplit == 1 or by combine)
  float* part;              // [B*Hq, nsplit, D+2] partial (m, l, acc)
  int k, d, nsplit, kc;
  int low_dim;              // logits from the leading d coordinates only (PCAAttn)
  float scale_log2;         // softmax scale * log2(e)
  Shape sh;
};

struct FusedParams {
  const void* q;        // [B,Hq,D]
  const void* k_new;    // [B,Hkv,D] nullable: appended as token S-1 when set
  const void* v_new;    // [B,Hkv,D]
  void* kcache;         // written only at row S-1, when appending
  void* vcache;
  const float* P;       // [Hkv,D,D]
  void* out;            // [B,Hq,D] in sh.odt
  int32_t* idx_out;     // [B,Hq,k] nullable
  int k;
  float scale_log2;
  int threads;          // workgroup size: 256 or 512
  // paired units (single head): helpers for units [help_first, help_first + n_help)
  int n_units;          // B * Hkv: workgroups with a unit of their own
  int help_first, n_help, k0;
  float* help_part;     // [n_help][2][D + 2] partials (coherent accesses only)
  unsigned long long* help_flag;  // [n_help] launch tag of the first half done
  unsigned long long tag;         // unique per launch on one workspace, nonzero
  Shape sh;
};

struct HeadParams {
  const void* q;        // [B,Hq,D]
  const void* k_new;    // [B,Hkv,D] nullable: appended as token S-1 when set
  const void* v_new;    // [B,Hkv,D]
  void* kcache;         // written only at row S-1, when appending
  void* vcache;
  const float* P;       // [Hkv,D,D]
  void* out;            // [B,Hq,D] in sh.odt
  int32_t* idx_out;     // [B,Hq,k] nullable
  int k;
  float scale_log2;
  int n_slots;          // workgroups of the heads (grouped heads: padded to whole XCD blocks)
  // paired heads (single query head per KV head): helpers for heads
  // [help_first, help_first + n_help), workgroups n_heads ...
  int n_heads;          // B * Hq
  int help_first, n_help, k0;
  float* help_part;     // [n_help][2][D + 2] partials (coherent accesses only)
  unsigned long long* help_flag;  // [n_help] launch tag of the first half done
  unsigned long long tag;         // unique per launch on one workspace, nonzero
  // a head and its helper sharing out the panel stream: each streams one
  // half of the passes and hands its scores over
  int share;                      // 1: the pairs share the stream
  float* xbuf;                    // [B*Hq][S] scores handed over (coherent accesses only)
  unsigned long long* xflag;      // [n_help][4] members' flags (tag), the first through at 2
  unsigned long long wait_ticks;  // longest wait for the partner's half (100 MHz clock)
  Shape sh;
};

struct PrefillParams {
  const void* k_rows;  // [B, Hkv, n_tokens, D] storage dtype, unrotated keys
  const float* P;      // [Hkv, D, D]
  void* kcache;        // split-panel layout, rows [pos, pos + n_tokens) written
  int n_tokens, pos;
  int cus;             // compute units of the device
  Shape sh;
};

struct CalibParams {
  const void* keys;     // [Hkv, n, D] storage dtype, unrotated calibration keys
  int n, nch;           // keys per head; chunks of kCalChunk keys
  float* part_s2;       // [Hkv, nch, D, D] partial sums of y y^T (y = key - first key)
  float* part_s1;       // [Hkv, nch, D] partial sums of y
  float* P;             // [Hkv, D, D] principal directions as columns
  float* variances;     // [Hkv, D] nullable
  Shape sh;
};

// Calibration keys summed by one covariance workgroup.
constexpr int kCalChunk = 2048;

struct LayoutParams {
  const void* src;
  void* dst;
  int n_tokens;
  int to_cache;  // 1: row-major -> cache layout, 0: cache -> row-major
  Shape sh;
};

hipError_t launch_project(const ProjectParams& p, hipStream_t st);
hipError_t launch_score(const ScoreParams& p, hipStream_t st);
// Workgroups of the panel score kernel with four lanes per token (its staged
// tiles) for this shape.
long long score_workgroups_staged(const Shape& sh);
hipError_t launch_topk(const TopkParams& p, int n_rows, hipStream_t st);
hipError_t launch_attend(const AttendParams& p, hipStream_t st);
hipError_t launch_layout(const LayoutParams& p, hipStream_t st);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t st);
hipError_t launch_calibrate(const CalibParams& p, hipStream_t st);

// One-launch decode step (rotation, scores, top-k, attention) for shapes whose
// per-unit scores fit the workgroup's LDS budget.
bool fused_supported(const Shape& sh, int d, int k);
hipError_t launch_fused(const FusedParams& p, hipStream_t st);

// One-launch decode step with one query head per workgroup and its whole row
// of scores in LDS (rows up to 32768 tokens), for shapes the kernel above
// does not take.
bool head_supported(const Shape& sh, int d, int k);
int head_kernel_threads(const Shape& sh);
// whether a head and its helper share out the stream of a row of `streamed`
// panel rows (each half at least two load batches)
bool head_share_ok(const Shape& sh, int streamed);
constexpr unsigned long long kShareWaitTicks = 2000;  // 20 us of the 100 MHz clock
hipError_t launch_head(const HeadParams& p, hipStream_t st);

// Rows of the selected set processed by one attention workgroup.
constexpr int kAttendChunk = 2048;    // most rows of one attention workgroup
constexpr int kAttendChunkMin = 512;  // fewest (when larger chunks would leave CUs idle)

}  // namespace loki
