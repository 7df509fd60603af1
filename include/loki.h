/*
 * loki.h -- C ABI of the Loki sparse decode-attention library for AMD MI355X
 * (gfx950 / CDNA4).
 *
 * Method: "Loki: Low-Rank Keys for Efficient Sparse Attention" (Singhania,
 * Singh, He, Feizi, Bhatele; NeurIPS 2024).  Keys are cached in a PCA basis
 * calibrated offline; each decode step rotates the query into that basis,
 * scores every cached token with the leading d principal components only,
 * keeps the top k tokens per (batch, query head) and runs exact softmax
 * attention with the full-dimensional keys over those k tokens.  Sources:
 *   [A]  briefgpt.xyz keyword page "loki" -- the paper's abstract: tokens are
 *        ranked and selected by attention scores computed in low-dimensional
 *        space;
 *   [T]  deep-diver.github.io NeurIPS-2024 poster page, "TL;DR": exact
 *        attention scores are computed just for the tokens that the
 *        low-dimensional ranking keeps;
 *   [F1] same page, "Visual Insights", Figure 1 (right): offline PCA of the
 *        keys, approximate scores in the low-dimensional space, top-k, final
 *        scores with the full-dimensional keys;
 *   [C]  same page, "In-depth insights", "Loki's Computational Cost": the
 *        KV-cache append is part of each step;
 *   [TB] same page, "More on tables", first table: k_f is the fraction of keys
 *        kept, d_f the fraction of the key dimensions used for scoring;
 *   [VA] same page, "More on figures": per-layer attention time of vanilla
 *        attention against Loki (Llama2-13B), the speed-up being measured;
 *   [PT] same page, "More on tables", the PCAAttn table: a Loki variant that
 *        attends with the reduced-dimensional scores directly;
 *   [FG] same page, "More on figures": the rank at which PCA of the keys
 *        explains 90% of their variance, and the offline PCA calibration step.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers, owned by the caller, at least
 *     16-byte aligned; the library never allocates or frees device memory
 *     and never synchronises.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; the call returns after enqueueing.
 *   - Arguments are validated before anything is enqueued: on any error
 *     nothing is launched and no output is written.  Return value 0 = OK,
 *     negative = loki_status; loki_last_error() gives a detail string
 *     (thread-local).  A launch failure reported by the HIP runtime returns
 *     LOKI_EHIP.
 *   - Calls that share a workspace must not overlap in time.
 *   - Host-side state: per device, the compute-unit count and the address of
 *     the no-alloc scratch array are cached on first use; per workspace
 *     pointer that a decode call used with paired workgroups, one 64-bit
 *     launch counter (16 bytes of host memory each, kept until the process
 *     ends, so a caller that cycles through many distinct workspaces grows
 *     that table by one entry per workspace).  No device memory is ever
 *     allocated.
 *
 * Layouts (element = the storage dtype of loki_desc.dtype)
 *   q        [B, Hq, D]
 *   V cache  [B, Hkv, S_cap, D] row-major
 *   K cache  rotated keys (k . P) in the split-panel layout: per (b, kv) one
 *            block of S_cap*D elements, first the leading dp coordinates of
 *            every token ([S_cap, dp], token-major), then the remaining D-dp
 *            coordinates ([S_cap, D-dp]).  Same size as a row-major cache.
 *            Written only through loki_pack_kcache, loki_prefill,
 *            loki_append and loki_decode_append.
 *   P        [Hkv, D, D] fp32 row-major; column j is the j-th principal
 *            direction (descending variance), so k_rot = k . P.  Query head h
 *            uses P[h / (Hq/Hkv)].
 *   qr       [B, Hq, D] fp32, scores [B, Hq, S] fp32, idx [B, Hq, k] int32,
 *   out      [B, Hq, D] in loki_desc.out_dtype (fp32 by default).
 */
#ifndef LOKI_H
#define LOKI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOKI_OK = 0,
  LOKI_EINVAL = -1,       /* argument outside its documented domain, null or misaligned pointer */
  LOKI_EUNSUPPORTED = -2, /* valid but not built: head_dim, panel width, GQA group size */
  LOKI_EWORKSPACE = -3,   /* workspace smaller than loki_workspace_bytes() */
  LOKI_EHIP = -4          /* the HIP runtime refused a launch */
} loki_status;

typedef enum { LOKI_F32 = 0, LOKI_F16 = 1, LOKI_BF16 = 2 } loki_dtype;

typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t n_q_heads;    /* Hq >= 1 */
  int32_t n_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0, Hq/Hkv in 1..16 */
  int32_t head_dim;     /* D: 64, 96 or 128 (the poster page's "More on figures"
                           studies models whose key heads have 96 as well as
                           128 dimensions) */
  int32_t seq_len;      /* S: tokens attended, 1 <= S <= seq_capacity */
  int32_t seq_capacity; /* S_cap: rows allocated per (b, kv) in both caches */
  int32_t panel_dim;    /* dp: leading rotated coordinates stored as the scoring
                           panel; a power of two, 16 <= dp*elem_bytes, dp <= D.
                           Scoring is fastest with d <= dp, the final attention
                           with d == dp. */
  int32_t dtype;        /* loki_dtype of q, K cache, V cache, k_new, v_new */
  float softmax_scale;  /* <= 0 selects 1/sqrt(D) */
  uint32_t flags;       /* LOKI_FLAG_* bits, 0 by default */
  int32_t out_dtype;    /* loki_dtype of every attention output `out`: LOKI_F32
                           (0, the default) or LOKI_F16 / LOKI_BF16, the fp32
                           result rounded to nearest-even once at the store */
} loki_desc;

/* loki_desc.flags: run a decode step as separate launches (query rotation,
   scores, top-k, attention) even where the one-launch kernel applies.  Same
   results up to fp32 summation order; for profiling the phases. */
#define LOKI_FLAG_SEPARATE_KERNELS 1u

/* loki_desc.flags: in the one-launch kernel, one workgroup per (b, kv) only.
   By default (single query head per KV head, k >= 256), when the (b, kv)
   units do not fill whole rounds of the compute units, spare workgroup slots
   run helpers: a helper repeats the selection of one of the units of the
   last round and attends the second half of its rows, and the two halves are
   merged (through the workspace).  Same index sets; outputs equal up to fp32
   summation order.  A captured launch replays correctly: the pair's flag is
   cleared by the second of the two. */
#define LOKI_FLAG_NO_HELPERS 2u

/* loki_desc.flags: in the one-launch kernel with one query head per
   workgroup, a head and its helper each stream the whole panel.  By default
   (rows of at least four load batches per half) each streams one half of the
   panel and the two hand their scores to each other through the workspace,
   so the panel is read once, with the nontemporal policy.  Same results, bit
   for bit. */
#define LOKI_FLAG_NO_SHARED_STREAM 4u

/* loki_desc.flags, for testing: the two workgroups sharing a stream do not
   wait for each other; a half that is not published when it is needed is
   scored by the workgroup that needs it (the path a workgroup takes when
   its partner is not resident within 20 us).  Same results, bit for bit. */
#define LOKI_FLAG_SHARED_NO_WAIT 8u

/* loki_desc.flags: take the one-launch kernel with one query head per
   workgroup (plan 2 of loki_decode_plan) also where the one with one
   workgroup per (b, kv) applies.  Same index sets; outputs equal up to fp32
   summation order. */
#define LOKI_FLAG_PER_HEAD_KERNEL 16u

/* Human-readable name of a status code; never NULL. */
const char* loki_strerror(int status);

/* Detail of the last failed call on this thread ("" if none). */
const char* loki_last_error(void);

/* Number of elements of the K cache (= B*Hkv*S_cap*D) for `desc`. */
int loki_kcache_elems(const loki_desc* desc, size_t* n_elems);

/* Bytes of workspace loki_decode / loki_decode_append need for (d, k). */
int loki_workspace_bytes(const loki_desc* desc, int d, int k, size_t* bytes);

/*
 * Launch plan of a decode step: *one_launch is nonzero when loki_decode
 * (append = 0) or loki_decode_append (append = 1) with these arguments runs as
 * a single kernel, 0 when it runs as separate launches (d != panel_dim, head
 * dimension 64, or LOKI_FLAG_SEPARATE_KERNELS).  1: one workgroup per
 * (b, kv) with its group's scores in LDS (head_dim 128, Hq/Hkv in {1, 2, 4},
 * S <= 4096, the group's scores and index lists within the LDS budget).
 * 2: otherwise, up to S = 32768: one workgroup per query head with its whole
 * row of scores in LDS (plus helper workgroups sharing the heads' panel
 * stream and attention when the heads leave compute units free).  The plan
 * is the same with or without append.
 */
int loki_decode_plan(const loki_desc* desc, int d, int k, int append, int* one_launch);

/*
 * Cache layout conversion.  krot_rows [B, Hkv, n_tokens, D] row-major rotated
 * keys <-> the first n_tokens rows of every (b, kv) block of the K cache.
 * n_tokens in [0, S_cap].  Pure data movement.
 */
int loki_pack_kcache(const void* krot_rows, int32_t n_tokens, void* kcache,
                     const loki_desc* desc, void* stream);
int loki_unpack_kcache(const void* kcache, int32_t n_tokens, void* krot_rows,
                       const loki_desc* desc, void* stream);

/*
 * Append one token per (b, kv) at row `pos` (0 <= pos < S_cap) [C], [F1]:
 * K cache row pos := round_to_dtype(k_new . P[kv]) (fp32 product, rounded to
 * nearest even), V cache row pos := v_new (copied).  k_new, v_new [B, Hkv, D].
 */
int loki_append(const void* k_new, const void* v_new, const float* P, void* kcache,
                void* vcache, int32_t pos, const loki_desc* desc, void* stream);

/*
 * Prefill [C], [F1]: the append of a whole run of tokens at once.  For
 * t < n_tokens, K cache row pos + t := round_to_dtype(k_rows[b,kv,t,:] . P[kv])
 * and, when v_rows is not NULL, V cache row pos + t := v_rows[b,kv,t,:]
 * (copied; vcache is then required).  k_rows, v_rows [B, Hkv, n_tokens, D] in
 * the storage dtype, unrotated; 0 <= pos, pos + n_tokens <= S_cap
 * (n_tokens = 0: nothing is enqueued).  The product is formed with fp32
 * accuracy: fp32 keys use fp32 arithmetic; fp16 / bf16 keys use matrix-core
 * products of the exact 16-bit keys with P split into two (fp16) or three
 * (bf16) 16-bit parts, accumulated in fp32.  Either way the stored value is
 * within one unit in the last place of the exact product rounded once.
 * Rows outside [pos, pos + n_tokens) are not touched.  k_rows must not
 * overlap the caches.
 */
int loki_prefill(const void* k_rows, const void* v_rows, int32_t n_tokens, int32_t pos,
                 const float* P, void* kcache, void* vcache, const loki_desc* desc, void* stream);

/* Query rotation [F1]: qr[b,h,:] = q[b,h,:] . P[h / (Hq/Hkv)] in fp32. */
int loki_rotate_query(const void* q, const float* P, float* qr, const loki_desc* desc,
                      void* stream);

/*
 * Approximate scores [A], [F1], [TB]:
 * scores[b,h,t] = sum_{j<d} qr[b,h,j] * krot[b,kv,t,j] for t < S, 1 <= d <= D.
 * No scaling.
 */
int loki_score(const float* qr, const void* kcache, int d, float* scores,
               const loki_desc* desc, void* stream);

/*
 * Top-k selection [A], [T], [TB]: idx[b,h,:] = the k tokens ranked first by
 * (score descending, token ascending), listed in ascending token order;
 * -0 ranks as +0.  1 <= k <= S.  Scores must not be NaN.  sel_out
 * (nullable, [B, Hq, k] fp32) receives the scores of the selected tokens in
 * the same order (-0 as +0).
 */
int loki_topk(const float* scores, int k, int32_t* idx, float* sel_out, const loki_desc* desc,
              void* stream);

/*
 * Exact attention over given token sets [T], [F1]:
 * z_t = scale * sum_{j<D} qr[b,h,j] krot[b,kv,t,j] for t in idx[b,h,:],
 * out[b,h,:] = sum_t softmax(z)_t V[b,kv,t,:].  Entries of idx outside
 * [0, S) contribute zero weight (all of them outside -> NaN row).
 * sel_scores (nullable, [B, Hq, k]): the partial logits sum_{j<dp} qr_j
 * krot_{t,j} of the listed tokens over the leading panel_dim coordinates (what
 * loki_score with d = panel_dim and loki_topk's sel_out give); when given, only
 * the remaining D - panel_dim key coordinates are read.
 * Needs loki_workspace_bytes(desc, D, k) bytes of workspace.
 */
int loki_attend(const float* qr, const void* kcache, const void* vcache, const int32_t* idx,
                const float* sel_scores, int k, void* out, const loki_desc* desc,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * One full Loki decode step [A], [T], [F1]: rotate q, score all S tokens
 * with the leading d coordinates, select the top k per (b, h), exact softmax
 * attention over them.  1 <= d <= D, 1 <= k <= S.  out [B, Hq, D] in
 * desc->out_dtype.  idx_out (nullable) receives the selected sets
 * [B, Hq, k] in ascending order.  scores_out (nullable, [B, Hq, S] fp32,
 * 16-byte aligned) receives the low-dimensional scores of every token, the
 * values the selection ranked; a call with scores_out runs as separate
 * launches (the one-launch kernel keeps its scores on chip), whatever
 * loki_decode_plan reports.
 */
int loki_decode(const void* q, const void* kcache, const void* vcache, const float* P, int d,
                int k, void* out, int32_t* idx_out, float* scores_out, const loki_desc* desc,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): loki_decode
 * with the workspace taken from a fixed scratch array inside the library
 * instead of a caller's buffer.  Same arguments, launches and results as
 * loki_decode, without `workspace` / `workspace_bytes`.  Nothing is allocated
 * or freed: each GPU the library runs on holds its own copy of the array,
 * LOKI_NOALLOC_SCRATCH_BYTES bytes, from the first call on that device until
 * the process ends.  A step whose loki_workspace_bytes(desc, d, k) exceeds
 * that size is refused with LOKI_EWORKSPACE before anything else is done.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on
 * one GPU (two streams, two threads) race and must not be made; use
 * loki_decode with distinct workspaces for those.
 */
#define LOKI_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int loki_decode_noalloc(const void* q, const void* kcache, const void* vcache, const float* P,
                        int d, int k, void* out, int32_t* idx_out, float* scores_out,
                        const loki_desc* desc, void* stream);

/*
 * Append then decode [C], [F1]: appends (k_new, v_new) at row pos = S-1 as
 * loki_append does, then runs loki_decode over the S tokens (the new one
 * included).  k_new, v_new [B, Hkv, D] storage dtype.  As separate launches
 * the append shares the query-rotation launch; as one launch (see
 * loki_decode_plan) the kernel rotates and writes row S-1 itself and scores
 * the new token from the rounded row it wrote.  Either way row S-1 of both
 * caches holds the appended token on return; the rotated key may differ from
 * loki_append's in the last place of an element (a different fp32 summation
 * order before the rounding).
 */
int loki_decode_append(const void* q, const void* k_new, const void* v_new, void* kcache,
                       void* vcache, const float* P, int d, int k, void* out,
                       int32_t* idx_out, float* scores_out, const loki_desc* desc,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dense decode attention over all S cached tokens, the baseline the pages
 * measure Loki against ([T] "TL;DR" and [VA]: speed-up of Loki's attention
 * over vanilla attention): qr = q . P[kv], z_t = scale * qr . krot_t over all
 * D coordinates of every token t < S, out = softmax(z) . V.  Because P is
 * orthonormal, qr . krot_t = q . k_t: this is ordinary full attention, read
 * from the same rotated cache.  out [B, Hq, D] in desc->out_dtype.  The sequence is
 * taken in chunks of 512 to 2048 tokens, one workgroup each; when a row has
 * several chunks their partial softmax states are merged by a second launch.
 * Needs loki_workspace_bytes(desc, D, seq_len) bytes of workspace.
 */
int loki_full_attention(const void* q, const void* kcache, const void* vcache, const float* P,
                        void* out, const loki_desc* desc, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * PCAAttn [PT]: the Loki variant that attends with the reduced-dimensional
 * scores directly.  qr = q . P[kv], z_t = scale * sum_{j<d} qr_j krot_{t,j}
 * for every token t < S (no selection), out = softmax(z) . V over all S
 * tokens.  1 <= d <= D; d = D gives loki_full_attention's result.  Reads the
 * leading d coordinates of each cached key (the panel when d <= panel_dim)
 * and every V row.  out [B, Hq, D] in desc->out_dtype.  Needs
 * loki_workspace_bytes(desc, D, seq_len) bytes of workspace.
 */
int loki_pca_attention(const void* q, const void* kcache, const void* vcache, const float* P,
                       int d, void* out, const loki_desc* desc, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Calibration [F1], [FG]: the offline PCA that yields P, run on the GPU.
 * keys [Hkv, n, D] in the storage dtype: n >= 1 unrotated calibration keys
 * per KV head (only n_kv_heads, head_dim and dtype of desc are used, the rest
 * must still be valid).  Per KV head: C = (1/n) sum_t (x_t - mu)(x_t - mu)^T,
 * its eigenvectors written as the columns of P [Hkv, D, D] (fp32, row-major,
 * the layout every other call takes), ordered by descending eigenvalue, each
 * signed so that its first largest-magnitude entry is positive; variances
 * (nullable, [Hkv, D] fp32) receives the eigenvalues in the same order.
 * Accuracy: covariance from exact three-part bf16 products accumulated in
 * fp32, eigenvectors by fp32 Jacobi rotations; an eigenvector whose
 * eigenvalue is close to another's is determined only as far as that gap
 * allows.  Needs loki_calibrate_workspace_bytes(desc, n) bytes of workspace.
 */
int loki_calibrate_workspace_bytes(const loki_desc* desc, int32_t n, size_t* bytes);
int loki_calibrate(const void* keys, int32_t n, float* P, float* variances,
                   const loki_desc* desc, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LOKI_H */
