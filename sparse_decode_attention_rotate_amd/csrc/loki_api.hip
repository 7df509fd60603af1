// extern "C" entry points of libloki: argument validation, workspace layout,
// and the launch sequence of one decode step.  See include/loki.h for the
// contract of each call.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <random>
#include <string>
#include <unordered_map>

#include "loki.h"
#include "loki_internal.h"

using namespace loki;

// Scratch of loki_decode_noalloc: device memory in the library's own code
// object, one copy per GPU, held until the process ends.  Its name is only a
// host-side stand-in for the array; host code reaches the memory through the
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = LOKI_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return LOKI_OK;
  return fail(LOKI_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == LOKI_F32 ? 4 : 2; }

#define REQUIRE_PTR(p)                                                             \
  do {                                                                             \
    if ((p) == nullptr) return fail(LOKI_EINVAL, "%s is NULL", #p);                \
    if (!aligned16(p)) return fail(LOKI_EINVAL, "%s is not 16-byte aligned", #p);  \
  } while (0)

int check_desc(const loki_desc* d, Shape* sh) {
  if (!d) return fail(LOKI_EINVAL, "desc is NULL");
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(LOKI_EINVAL, "batch, n_q_heads and n_kv_heads must be >= 1");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(LOKI_EINVAL, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                d->n_q_heads, d->n_kv_heads);
  const int g = d->n_q_heads / d->n_kv_heads;
  if (g > 16) return fail(LOKI_EUNSUPPORTED, "query heads per KV head (%d) above 16", g);
  if (d->dtype != LOKI_F32 && d->dtype != LOKI_F16 && d->dtype != LOKI_BF16)
    return fail(LOKI_EINVAL, "dtype %d is not a loki_dtype", d->dtype);
  if (d->out_dtype != LOKI_F32 && d->out_dtype != LOKI_F16 && d->out_dtype != LOKI_BF16)
    return fail(LOKI_EINVAL, "out_dtype %d is not a loki_dtype", d->out_dtype);
  if (d->head_dim != 64 && d->head_dim != 96 && d->head_dim != 128)
    return fail(LOKI_EUNSUPPORTED, "head_dim %d (built: 64, 96, 128)", d->head_dim);
  if (d->seq_len < 1 || d->seq_capacity < d->seq_len || d->seq_capacity > (1 << 30))
    return fail(LOKI_EINVAL, "need 1 <= seq_len (%d) <= seq_capacity (%d) <= 2^30",
                d->seq_len, d->seq_capacity);
  const int dp = d->panel_dim, eb = elem_bytes(d->dtype);
  // one (b, kv) block of either cache is addressed with 32-bit byte offsets
  if ((size_t)d->seq_capacity * d->head_dim * eb >= ((size_t)1 << 31))
    return fail(LOKI_EUNSUPPORTED, "seq_capacity %d: one head's cache exceeds 2 GiB",
                d->seq_capacity);
  if (dp < 1 || dp > d->head_dim || (dp & (dp - 1)) != 0 || dp * eb < 16)
    return fail(LOKI_EINVAL,
                "panel_dim %d must be a power of two <= head_dim with panel_dim*elem >= 16", dp);
  sh->B = d->batch;
  sh->Hq = d->n_q_heads;
  sh->Hkv = d->n_kv_heads;
  sh->g = g;
  sh->D = d->head_dim;
  sh->S = d->seq_len;
  sh->S_cap = d->seq_capacity;
  sh->dp = dp;
  sh->dtype = d->dtype;
  sh->odt = d->out_dtype;
  sh->kl.head_elems = (size_t)d->seq_capacity * d->head_dim;
  sh->kl.rest_off = (size_t)d->seq_capacity * dp;
  sh->kl.dp = dp;
  sh->kl.rest = d->head_dim - dp;
  return LOKI_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t qr, scores, idx, sel, part, help_flag, help_part, xflag, total;
  int nsplit;
};

WsLayout ws_layout(const Shape& sh, int k) {
  WsLayout w;
  const size_t units = (size_t)sh.B * sh.Hq;
  // partials for the smaller chunk: either chunk size fits (attend_plan)
  w.nsplit = (k + kAttendChunkMin - 1) / kAttendChunkMin;
  size_t off = 0;
  w.qr = off;
  off += align256(units * sh.D * 4);
  w.scores = off;
  off += align256(units * sh.S * 4);
  w.idx = off;
  off += align256(units * (size_t)k * 4);
  w.sel = off;
  off += align256(units * (size_t)k * 4);
  w.part = off;
  off += w.nsplit > 1 ? align256(units * w.nsplit * (size_t)(sh.D + 2) * 4) : 0;
  // paired units of the one-launch kernel: one flag and two partials per (b, kv)
  const size_t kv_units = (size_t)sh.B * sh.Hkv;
  w.help_flag = off;
  off += align256(kv_units * 8);
  w.help_part = off;
  off += align256(kv_units * 2 * (size_t)(sh.D + 2) * 4);
  // pairs of the one-head-per-workgroup kernel sharing the stream: four
  // words per pair (at most one pair per query head); the scores handed over
  // go through the scores region
  w.xflag = off;
  off += align256(units * 4 * 8);
  w.total = off;
  return w;
}

// Launch tags of the paired units, per workspace: a pair's flag holds the tag
// of the launch that last used it, so stale flags never match a later launch
// and need no reset; a random start makes a match with whatever an earlier
// process left in the memory unlikely (64-bit tags).
unsigned long long next_tag(const void* workspace) {
  static std::mutex mu;
  static std::unordered_map<const void*, unsigned long long> tags;
  std::lock_guard<std::mutex> lock(mu);
  auto it = tags.find(workspace);
  if (it == tags.end()) {
    std::random_device rd;
    const unsigned long long start = ((unsigned long long)rd() << 32) ^ rd();
    it = tags.emplace(workspace, start).first;
  }
  if (++it->second == 0) ++it->second;
  return it->second;
}

// Compute units of the current device (cached per device).
int compute_units() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Rows per attention workgroup (512, 1024 or 2048) for k rows per query
// head.  One split -- no merge launch -- when the rows alone give a workgroup
// per compute unit; else the largest chunk that still gives two per compute
// unit (fewer splits to merge, fewer workgroups to start); else 512.  Sets
// ap.kc and ap.nsplit.
void attend_plan(AttendParams& ap, const Shape& sh, int k) {
  const long long rows = (long long)sh.B * sh.Hq;
  const int cu = compute_units();
  ap.kc = kAttendChunkMin;
  if (k <= kAttendChunk && rows >= cu) {
    while (ap.kc < k) ap.kc *= 2;
  } else {
    for (int c = kAttendChunk; c > kAttendChunkMin; c /= 2)
      if (rows * ((k + c - 1) / c) >= 2LL * cu) {
        ap.kc = c;
        break;
      }
  }
  ap.nsplit = (k + ap.kc - 1) / ap.kc;
}

float scale_log2(const loki_desc* d) {
  const float s = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  return s * 1.4426950408889634f;  // log2(e)
}

int decode_impl(const void* q, const void* k_new, const void* v_new, void* kcache, void* vcache,
                const float* P, int d, int k, void* out, int32_t* idx_out, float* scores_out,
                const loki_desc* desc, void* workspace, size_t workspace_bytes, void* stream,
                bool append) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  REQUIRE_PTR(q);
  REQUIRE_PTR(kcache);
  REQUIRE_PTR(vcache);
  REQUIRE_PTR(P);
  REQUIRE_PTR(out);
  REQUIRE_PTR(workspace);
  if (append) {
    REQUIRE_PTR(k_new);
    REQUIRE_PTR(v_new);
  }
  if (idx_out && !aligned16(idx_out)) return fail(LOKI_EINVAL, "idx_out is not 16-byte aligned");
  if (scores_out && !aligned16(scores_out))
    return fail(LOKI_EINVAL, "scores_out is not 16-byte aligned");
  if (d < 1 || d > sh.D) return fail(LOKI_EINVAL, "d = %d outside [1, %d]", d, sh.D);
  if (k < 1 || k > sh.S) return fail(LOKI_EINVAL, "k = %d outside [1, %d]", k, sh.S);
  const WsLayout w = ws_layout(sh, k);
  if (workspace_bytes < w.total)
    return fail(LOKI_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, w.total);

  hipStream_t st = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  float* qr = reinterpret_cast<float*>(ws + w.qr);
  float* scores = scores_out ? scores_out : reinterpret_cast<float*>(ws + w.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + w.idx);
  const bool split = (d == sh.dp);
  float* sel = split ? reinterpret_cast<float*>(ws + w.sel) : nullptr;

  // the one-launch kernel keeps the scores on chip: a call that asks for
  // them takes the separate launches
  if (!scores_out && !(desc->flags & (LOKI_FLAG_SEPARATE_KERNELS | LOKI_FLAG_PER_HEAD_KERNEL)) &&
      fused_supported(sh, d, k)) {
    FusedParams fp{};
    fp.q = q;
    fp.k_new = append ? k_new : nullptr;
    fp.v_new = append ? v_new : nullptr;
    fp.kcache = kcache;
    fp.vcache = vcache;
    fp.P = P;
    fp.out = out;
    fp.idx_out = idx_out;
    fp.k = k;
    fp.scale_log2 = scale_log2(desc);
    fp.sh = sh;
    // one workgroup per (b, kv): with no more of them than compute units, use
    // 512 threads so that each unit has twice the loads in flight
    const int units = sh.B * sh.Hkv, ncu = compute_units();
    fp.threads = units <= ncu ? 512 : 256;
    fp.n_units = units;
    // Paired units: when the units do not fill whole rounds of one workgroup
    // per compute unit, the last (partial) round leaves some compute units
    // with one unit more than the others.  Up to as many helper workgroups as
    // that round has free slots take the second half of the attention of
    // those units (k >= 256, single head); a multiple of 8 keeps a helper on
    // the same die (L2) as its unit, whose panel it re-reads.
    const int per_cu = fp.threads == 256 ? 3 : 2;  // resident workgroups per CU
    const int full = units / ncu, part = units % ncu;
    int n_help = 0;
    if (sh.g == 1 && k >= 256 && part > 0 && full + 1 <= per_cu &&
        !(desc->flags & LOKI_FLAG_NO_HELPERS))
      n_help = (part < ncu - part ? part : ncu - part) / 8 * 8;
    fp.n_help = n_help;
    fp.help_first = units - n_help;
    fp.k0 = (k / 2 + 63) / 64 * 64;
    if (n_help > 0) {
      fp.help_part = reinterpret_cast<float*>(ws + w.help_part);
      fp.help_flag = reinterpret_cast<unsigned long long*>(ws + w.help_flag);
      fp.tag = next_tag(workspace);
    }
    return hip_status(launch_fused(fp, st), "fused");
  }
  // Longer rows (up to 32768 tokens), or grouped heads whose scores do not
  // fit one workgroup: the one-launch kernel with one query head per
  // workgroup and its row of scores in LDS.
  if (!scores_out && !(desc->flags & LOKI_FLAG_SEPARATE_KERNELS) && head_supported(sh, d, k)) {
    HeadParams hp{};
    hp.q = q;
    hp.k_new = append ? k_new : nullptr;
    hp.v_new = append ? v_new : nullptr;
    hp.kcache = kcache;
    hp.vcache = vcache;
    hp.P = P;
    hp.out = out;
    hp.idx_out = idx_out;
    hp.k = k;
    hp.scale_log2 = scale_log2(desc);
    hp.sh = sh;
    const int heads = sh.B * sh.Hq;
    hp.n_heads = heads;
    if (sh.g == 1) {
      hp.n_slots = heads;
      // Paired heads: while the heads leave resident workgroup slots free
      // (two per compute unit at 512 threads, one at 1024), up to as many
      // helpers as free slots (a multiple of 8, so that a helper and its
      // head share one XCD's L2) attend the second half of a head's rows.
      const int slots = compute_units() * (head_kernel_threads(sh) == 512 ? 2 : 1);
      int n_help = 0;
      if (k >= 256 && heads < slots && !(desc->flags & LOKI_FLAG_NO_HELPERS))
        n_help = (heads < slots - heads ? heads : slots - heads) / 8 * 8;
      hp.n_help = n_help;
      hp.help_first = heads - n_help;
      hp.k0 = (k / 2 + 63) / 64 * 64;
      if (n_help > 0) {
        hp.help_part = reinterpret_cast<float*>(ws + w.help_part);
        hp.help_flag = reinterpret_cast<unsigned long long*>(ws + w.help_flag);
        hp.tag = next_tag(workspace);
        // a head and its helper stream one half of the panel each and hand
        // the scores over (every workgroup is resident at once: heads +
        // helpers <= slots)
        if (!(desc->flags & LOKI_FLAG_NO_SHARED_STREAM) &&
            head_share_ok(sh, append ? sh.S - 1 : sh.S)) {
          hp.share = 1;
          hp.xbuf = reinterpret_cast<float*>(ws + w.scores);
          hp.xflag = reinterpret_cast<unsigned long long*>(ws + w.xflag);
          hp.wait_ticks = (desc->flags & LOKI_FLAG_SHARED_NO_WAIT) ? 0ull : kShareWaitTicks;
        }
      }
    } else {
      // the g heads of a (b, kv) on one XCD: whole blocks of 8 (b, kv) units
      hp.n_slots = (sh.B * sh.Hkv + 7) / 8 * 8 * sh.g;
      hp.help_first = heads;
    }
    return hip_status(launch_head(hp, st), "head");
  }

  // For the score kernel's staged tiles (head_dim 128, four lanes per token,
  // 1, 2 or 4 query heads per KV head), the score kernel can rotate the query
  // itself, write qr for the attention and do the append: no separate
  // rotation launch.  Every score workgroup repeats the rotation of its heads'
  // panel coordinates, which pays when the grid is one round of resident
  // workgroups (four per compute unit), not when its tiles make several
  // rounds (measured: 13B separate step 79.5 -> 71.4 us; GQA, 2048
  // workgroups, 140.4 -> 142.2 us).
  const int lpt = sh.dp * elem_bytes(sh.dtype) / 16;
  const bool rotate_in_score = sh.D == 128 && lpt == 4 && d <= sh.dp &&
                               (sh.g == 1 || sh.g == 2 || sh.g == 4) &&
                               score_workgroups_staged(sh) <= 4LL * compute_units();
  if (!rotate_in_score) {
    ProjectParams pp{};
    pp.q = q;
    pp.k_new = append ? k_new : nullptr;
    pp.v_new = append ? v_new : nullptr;
    pp.P = P;
    pp.qr = qr;
    pp.kcache = kcache;
    pp.vcache = vcache;
    pp.pos = sh.S - 1;
    pp.sh = sh;
    if ((rc = hip_status(launch_project(pp, st), "project"))) return rc;
  }

  ScoreParams sp{};
  sp.qr = qr;
  if (rotate_in_score) {
    sp.q = q;
    sp.P = P;
    sp.qr_out = qr;
    if (append) {
      sp.k_new = k_new;
      sp.v_new = v_new;
      sp.kcache_w = kcache;
      sp.vcache_w = vcache;
    }
  }
  sp.kcache = kcache;
  sp.scores = scores;
  sp.d = d;
  sp.sh = sh;
  if ((rc = hip_status(launch_score(sp, st), "score"))) return rc;

  TopkParams tp{};
  tp.scores = scores;
  tp.idx = idx;
  tp.sel_scores = sel;
  tp.S = sh.S;
  tp.k = k;
  if ((rc = hip_status(launch_topk(tp, sh.B * sh.Hq, st), "topk"))) return rc;

  AttendParams ap{};
  ap.qr = qr;
  ap.kcache = kcache;
  ap.vcache = vcache;
  ap.idx = idx;
  ap.sel_scores = sel;
  ap.out = out;
  ap.part = reinterpret_cast<float*>(ws + w.part);
  ap.k = k;
  ap.d = d;
  attend_plan(ap, sh, ap.k);
  ap.scale_log2 = scale_log2(desc);
  ap.sh = sh;
  return hip_status(launch_attend(ap, st), "attend");
}

int scratch_address(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(LOKI_EUNSUPPORTED, "device %d: at most 64 devices", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(LOKI_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return LOKI_OK;
}

}  // namespace

extern "C" {

const char* loki_strerror(int status) {
  switch (status) {
    case LOKI_OK: return "ok";
    case LOKI_EINVAL: return "invalid argument";
    case LOKI_EUNSUPPORTED: return "unsupported configuration";
    case LOKI_EWORKSPACE: return "workspace too small";
    case LOKI_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* loki_last_error(void) { return g_last_error.c_str(); }

int loki_kcache_elems(const loki_desc* desc, size_t* n_elems) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  if (!n_elems) return fail(LOKI_EINVAL, "n_elems is NULL");
  *n_elems = (size_t)sh.B * sh.Hkv * sh.kl.head_elems;
  return LOKI_OK;
}

int loki_workspace_bytes(const loki_desc* desc, int d, int k, size_t* bytes) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  if (!bytes) return fail(LOKI_EINVAL, "bytes is NULL");
  if (d < 1 || d > sh.D) return fail(LOKI_EINVAL, "d = %d outside [1, %d]", d, sh.D);
  if (k < 1 || k > sh.S) return fail(LOKI_EINVAL, "k = %d outside [1, %d]", k, sh.S);
  *bytes = ws_layout(sh, k).total;
  return LOKI_OK;
}

int loki_decode_plan(const loki_desc* desc, int d, int k, int append, int* one_launch) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  if (!one_launch) return fail(LOKI_EINVAL, "one_launch is NULL");
  if (d < 1 || d > sh.D) return fail(LOKI_EINVAL, "d = %d outside [1, %d]", d, sh.D);
  if (k < 1 || k > sh.S) return fail(LOKI_EINVAL, "k = %d outside [1, %d]", k, sh.S);
  (void)append;  // the one-launch kernel appends too
  *one_launch = 0;
  if (!(desc->flags & LOKI_FLAG_SEPARATE_KERNELS))
    *one_launch = fused_supported(sh, d, k) && !(desc->flags & LOKI_FLAG_PER_HEAD_KERNEL)
                      ? 1
                      : (head_supported(sh, d, k) ? 2 : 0);
  return LOKI_OK;
}

static int layout_impl(const void* src, void* dst, int32_t n_tokens, const loki_desc* desc,
                       void* stream, int to_cache) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  REQUIRE_PTR(src);
  REQUIRE_PTR(dst);
  if (n_tokens < 0 || n_tokens > sh.S_cap)
    return fail(LOKI_EINVAL, "n_tokens = %d outside [0, %d]", n_tokens, sh.S_cap);
  LayoutParams p{};
  p.src = src;
  p.dst = dst;
  p.n_tokens = n_tokens;
  p.to_cache = to_cache;
  p.sh = sh;
  return hip_status(launch_layout(p, (hipStream_t)stream), "layout");
}

int loki_pack_kcache(const void* krot_rows, int32_t n_tokens, void* kcache,
                     const loki_desc* desc, void* stream) {
  return layout_impl(krot_rows, kcache, n_tokens, desc, stream, 1);
}

int loki_unpack_kcache(const void* kcache, int32_t n_tokens, void* krot_rows,
                       const loki_desc* desc, void* stream) {
  return layout_impl(kcache, krot_rows, n_tokens, desc, stream, 0);
}

int loki_append(const void* k_new, const void* v_new, const float* P, void* kcache,
                void* vcache, int32_t pos, const loki_desc* desc, void* stream) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  REQUIRE_PTR(k_new);
  REQUIRE_PTR(v_new);
  REQUIRE_PTR(P);
  REQUIRE_PTR(kcache);
  REQUIRE_PTR(vcache);
  if (pos < 0 || pos >= sh.S_cap) return fail(LOKI_EINVAL, "pos = %d outside [0, %d)", pos, sh.S_cap);
  ProjectParams pp{};
  pp.k_new = k_new;
  pp.v_new = v_new;
  pp.P = P;
  pp.kcache = kcache;
  pp.vcache = vcache;
  pp.pos = pos;
  pp.sh = sh;
  return hip_status(launch_project(pp, (hipStream_t)stream), "append");
}

int loki_prefill(const void* k_rows, const void* v_rows, int32_t n_tokens, int32_t pos,
                 const float* P, void* kcache, void* vcache, const loki_desc* desc, void* stream) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  REQUIRE_PTR(k_rows);
  REQUIRE_PTR(P);
  REQUIRE_PTR(kcache);
  if (v_rows) REQUIRE_PTR(vcache);
  if (n_tokens < 0 || pos < 0 || (int64_t)pos + n_tokens > sh.S_cap)
    return fail(LOKI_EINVAL, "rows [%d, %d + %d) outside [0, %d)", pos, pos, n_tokens, sh.S_cap);
  if (n_tokens == 0) return LOKI_OK;
  hipStream_t st = (hipStream_t)stream;
  PrefillParams pp{};
  pp.k_rows = k_rows;
  pp.P = P;
  pp.kcache = kcache;
  pp.n_tokens = n_tokens;
  pp.pos = pos;
  pp.cus = compute_units();
  pp.sh = sh;
  rc = hip_status(launch_prefill(pp, st), "prefill");
  if (rc || !v_rows) return rc;
  // V rows are stored as given: one strided copy of B*Hkv blocks of n_tokens rows
  const size_t row = (size_t)sh.D * elem_bytes(sh.dtype);
  return hip_status(hipMemcpy2DAsync(static_cast<char*>(vcache) + (size_t)pos * row,
                                     (size_t)sh.S_cap * row, v_rows, (size_t)n_tokens * row,
                                     (size_t)n_tokens * row, (size_t)sh.B * sh.Hkv,
                                     hipMemcpyDeviceToDevice, st),
                    "prefill V copy");
}

int loki_rotate_query(const void* q, const float* P, float* qr, const loki_desc* desc,
                      void* stream) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  REQUIRE_PTR(q);
  REQUIRE_PTR(P);
  REQUIRE_PTR(qr);
  ProjectParams pp{};
  pp.q = q;
  pp.P = P;
  pp.qr = qr;
  pp.sh = sh;
  return hip_status(launch_project(pp, (hipStream_t)stream), "rotate_query");
}

int loki_score(const float* qr, const void* kcache, int d, float* scores, const loki_desc* desc,
               void* stream) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  REQUIRE_PTR(qr);
  REQUIRE_PTR(kcache);
  REQUIRE_PTR(scores);
  if (d < 1 || d > sh.D) return fail(LOKI_EINVAL, "d = %d outside [1, %d]", d, sh.D);
  ScoreParams sp{};
  sp.qr = qr;
  sp.kcache = kcache;
  sp.scores = scores;
  sp.d = d;
  sp.sh = sh;
  return hip_status(launch_score(sp, (hipStream_t)stream), "score");
}

int loki_topk(const float* scores, int k, int32_t* idx, float* sel_out, const loki_desc* desc,
              void* stream) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  REQUIRE_PTR(scores);
  REQUIRE_PTR(idx);
  if (k < 1 || k > sh.S) return fail(LOKI_EINVAL, "k = %d outside [1, %d]", k, sh.S);
  TopkParams tp{};
  if (sel_out && !aligned16(sel_out)) return fail(LOKI_EINVAL, "sel_out is not 16-byte aligned");
  tp.scores = scores;
  tp.idx = idx;
  tp.sel_scores = sel_out;
  tp.S = sh.S;
  tp.k = k;
  return hip_status(launch_topk(tp, sh.B * sh.Hq, (hipStream_t)stream), "topk");
}

int loki_attend(const float* qr, const void* kcache, const void* vcache, const int32_t* idx,
                const float* sel_scores, int k, void* out, const loki_desc* desc,
                void* workspace, size_t workspace_bytes, void* stream) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  REQUIRE_PTR(qr);
  REQUIRE_PTR(kcache);
  REQUIRE_PTR(vcache);
  REQUIRE_PTR(idx);
  REQUIRE_PTR(out);
  REQUIRE_PTR(workspace);
  if (k < 1 || k > sh.S) return fail(LOKI_EINVAL, "k = %d outside [1, %d]", k, sh.S);
  const WsLayout w = ws_layout(sh, k);
  if (workspace_bytes < w.total)
    return fail(LOKI_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, w.total);
  AttendParams ap{};
  if (sel_scores && !aligned16(sel_scores))
    return fail(LOKI_EINVAL, "sel_scores is not 16-byte aligned");
  ap.qr = qr;
  ap.kcache = kcache;
  ap.vcache = vcache;
  ap.idx = idx;
  ap.sel_scores = sel_scores;
  ap.out = out;
  ap.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.part);
  ap.k = k;
  ap.d = sel_scores ? sh.dp : sh.D;
  attend_plan(ap, sh, ap.k);
  ap.scale_log2 = scale_log2(desc);
  ap.sh = sh;
  return hip_status(launch_attend(ap, (hipStream_t)stream), "attend");
}

int loki_decode(const void* q, const void* kcache, const void* vcache, const float* P, int d,
                int k, void* out, int32_t* idx_out, float* scores_out, const loki_desc* desc,
                void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, nullptr, nullptr, const_cast<void*>(kcache), const_cast<void*>(vcache),
                     P, d, k, out, idx_out, scores_out, desc, workspace, workspace_bytes, stream,
                     false);
}

int loki_decode_append(const void* q, const void* k_new, const void* v_new, void* kcache,
                       void* vcache, const float* P, int d, int k, void* out,
                       int32_t* idx_out, float* scores_out, const loki_desc* desc,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, k_new, v_new, kcache, vcache, P, d, k, out, idx_out, scores_out, desc,
                     workspace, workspace_bytes, stream, true);
}

int loki_decode_noalloc(const void* q, const void* kcache, const void* vcache, const float* P,
                        int d, int k, void* out, int32_t* idx_out, float* scores_out,
                        const loki_desc* desc, void* stream) {
  // the size check comes first: an oversized call is refused before any HIP call
  size_t need = 0;
  int rc = loki_workspace_bytes(desc, d, k, &need);
  if (rc) return rc;
  if (need > kScratchBytes)
    return fail(LOKI_EWORKSPACE,
                "loki_decode_noalloc: this step needs %zu bytes of scratch, above the "
                "library's fixed %zu bytes; use loki_decode with a workspace",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return decode_impl(q, nullptr, nullptr, const_cast<void*>(kcache), const_cast<void*>(vcache),
                     P, d, k, out, idx_out, scores_out, desc, ws, kScratchBytes, stream, false);
}

// Dense (low_dim = 0) or low-dimensional (PCAAttn) attention over all S
// tokens: query rotation, then the split attention with identity rows.
static int all_tokens_attention(const void* q, const void* kcache, const void* vcache,
                                const float* P, int d, int low_dim, void* out,
                                const loki_desc* desc, void* workspace, size_t workspace_bytes,
                                void* stream, const char* what) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  REQUIRE_PTR(q);
  REQUIRE_PTR(kcache);
  REQUIRE_PTR(vcache);
  REQUIRE_PTR(P);
  REQUIRE_PTR(out);
  REQUIRE_PTR(workspace);
  if (d < 1 || d > sh.D) return fail(LOKI_EINVAL, "%s: d = %d outside [1, %d]", what, d, sh.D);
  const WsLayout w = ws_layout(sh, sh.S);
  if (workspace_bytes < w.total)
    return fail(LOKI_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, w.total);
  hipStream_t st = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  float* qr = reinterpret_cast<float*>(ws + w.qr);

  ProjectParams pp{};
  pp.q = q;
  pp.P = P;
  pp.qr = qr;
  pp.kcache = const_cast<void*>(kcache);
  pp.vcache = const_cast<void*>(vcache);
  pp.sh = sh;
  if ((rc = hip_status(launch_project(pp, st), "project"))) return rc;

  AttendParams ap{};
  ap.qr = qr;
  ap.kcache = kcache;
  ap.vcache = vcache;
  ap.idx = nullptr;  // every cached token
  ap.sel_scores = nullptr;
  ap.out = out;
  ap.part = reinterpret_cast<float*>(ws + w.part);
  ap.k = sh.S;
  ap.d = d;
  ap.low_dim = low_dim;
  attend_plan(ap, sh, ap.k);
  ap.scale_log2 = scale_log2(desc);
  ap.sh = sh;
  return hip_status(launch_attend(ap, st), what);
}

int loki_full_attention(const void* q, const void* kcache, const void* vcache, const float* P,
                        void* out, const loki_desc* desc, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const int D = desc ? desc->head_dim : 1;
  return all_tokens_attention(q, kcache, vcache, P, D, 0, out, desc, workspace, workspace_bytes,
                              stream, "full_attention");
}

int loki_pca_attention(const void* q, const void* kcache, const void* vcache, const float* P,
                       int d, void* out, const loki_desc* desc, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return all_tokens_attention(q, kcache, vcache, P, d, 1, out, desc, workspace, workspace_bytes,
                              stream, "pca_attention");
}

static size_t calib_part_bytes(const Shape& sh, int n, int* nch) {
  *nch = (n + kCalChunk - 1) / kCalChunk;
  return align256((size_t)sh.Hkv * *nch * sh.D * sh.D * 4);
}

int loki_calibrate_workspace_bytes(const loki_desc* desc, int32_t n, size_t* bytes) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  if (!bytes) return fail(LOKI_EINVAL, "bytes is NULL");
  if (n < 1) return fail(LOKI_EINVAL, "n = %d calibration keys (need >= 1)", n);
  int nch = 0;
  *bytes = calib_part_bytes(sh, n, &nch) + align256((size_t)sh.Hkv * nch * sh.D * 4);
  return LOKI_OK;
}

int loki_calibrate(const void* keys, int32_t n, float* P, float* variances,
                   const loki_desc* desc, void* workspace, size_t workspace_bytes, void* stream) {
  Shape sh;
  int rc = check_desc(desc, &sh);
  if (rc) return rc;
  REQUIRE_PTR(keys);
  REQUIRE_PTR(P);
  REQUIRE_PTR(workspace);
  if (variances && !aligned16(variances)) return fail(LOKI_EINVAL, "variances is not 16-byte aligned");
  if (n < 1) return fail(LOKI_EINVAL, "n = %d calibration keys (need >= 1)", n);
  size_t need = 0;
  if ((rc = loki_calibrate_workspace_bytes(desc, n, &need))) return rc;
  if (workspace_bytes < need)
    return fail(LOKI_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  CalibParams cp{};
  cp.keys = keys;
  cp.n = n;
  const size_t s1_off = calib_part_bytes(sh, n, &cp.nch);
  cp.part_s2 = static_cast<float*>(workspace);
  cp.part_s1 = reinterpret_cast<float*>(static_cast<char*>(workspace) + s1_off);
  cp.P = P;
  cp.variances = variances;
  cp.sh = sh;
  return hip_status(launch_calibrate(cp, (hipStream_t)stream), "calibrate");
}

}  // extern "C"
