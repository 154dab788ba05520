/*
 * lowram.h — C ABI of the LowRAM decode-step library (gfx950 / MI355X).
 *
 * One call runs the decode-time attention of one layer for a batch of
 * sequences against their compressed KV cache, as the LowRAM pages describe
 * it: the prefix is cut into chunks of S tokens whose mean post-RoPE key is a
 * landmark; each step scores the current query against the landmarks, keeps
 * the top-k chunks per KV head, rebuilds only those chunks' keys from
 * cross-layer low-rank coefficients times the layer-group basis and rotates
 * them at their token positions, predicts their values with the per-head
 * key-to-value MLP plus the stored residuals of the worst-predicted tokens,
 * and attends over them and the exact recent window.
 *   - LowRAM review (agihunt.info), key paragraph: xKV shared basis, RoPE
 *     undone before compression, chunked prefix, mean-key landmarks, top-k
 *     chunks rebuilt per query.
 *   - LowRAM explainer (cctest.ai), "How the method works": low-rank keys,
 *     amortised values, residuals for difficult tokens, selective
 *     reconstruction.
 *   - LowRAM abstract: a selected subset of KV pairs rebuilt per step.
 *
 * Conventions for every entry point
 *   - Array arguments are DEVICE pointers; the caller owns them.  The library
 *     never allocates, frees or synchronises: all work is enqueued on
 *     `stream` (a hipStream_t; NULL = the null stream) and returns at once.
 *   - bf16 and fp16 values travel as uint16_t bit patterns.
 *   - Arrays are dense, row-major, batch-major, in the layouts stated below,
 *     sliced to ONE layer by the caller.
 *   - Bulk arrays must be 16-byte aligned; int32/fp16 side arrays 4-byte.
 *   - Status: 0 on success, a negative LOWRAM_ERR_* otherwise.  Argument
 *     errors (NULL, SHAPE, UNSUPPORTED, WORKSPACE, ALIGN) are detected before
 *     any HIP call; LOWRAM_ERR_HIP reports a failed launch.
 *   - Calls are re-entrant for distinct workspaces; two calls that share a
 *     workspace must be ordered on one stream.
 */
#ifndef LOWRAM_H
#define LOWRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOWRAM_ABI_VERSION 3

enum {
  LOWRAM_OK = 0,
  LOWRAM_ERR_NULL = -1,        /* a required pointer is NULL                         */
  LOWRAM_ERR_SHAPE = -2,       /* inconsistent sizes (e.g. Hq % Hkv, P % S, k < 1)   */
  LOWRAM_ERR_UNSUPPORTED = -3, /* valid but not built (d != 128, S != 8, H != 256,
                                  or a grid past HIP's limits: more than 65535 in
                                  a y/z dimension, or more than (2^32 - 1) / 256
                                  workgroups of 256 work-items in a 1-D grid) */
  LOWRAM_ERR_WORKSPACE = -4,   /* workspace smaller than *_workspace_bytes reports    */
  LOWRAM_ERR_ALIGN = -5,       /* misaligned pointer                                 */
  LOWRAM_ERR_HIP = -6,         /* a HIP launch failed                                */
  LOWRAM_ERR_SCRATCH = -7      /* lowram_decode_step_noalloc: the shape needs more
                                  workspace than LOWRAM_NOALLOC_SCRATCH_BYTES       */
};

/* Size of the fixed device scratch of lowram_decode_step_noalloc: 64 MiB per
   GPU the library runs on, held from the library's load to the end of the
   process. */
#define LOWRAM_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Storage format of the coefficients C and of the residual values. */
enum {
  LOWRAM_FMT_BF16 = 0,
  /* int4 symmetric per group of 32 along the last axis: codes in [-7, 7],
     two per byte (even element in the low nibble, two's complement), one
     fp16 scale per group; value = float(code) * float(scale).  This is the
     quantised composition (LowRAM-Q / -EQ) of the LowRAM review's tables. */
  LOWRAM_FMT_INT4_G32 = 1
};

/* Sizes of one layer's decode step. */
typedef struct lowram_shape {
  int32_t batch;         /* 1 <= NB <= 65535 sequences                               */
  int32_t prefix_len;    /* P >= 0 compressed tokens, a multiple of chunk            */
  int32_t window;        /* W >= 0 exact recent tokens at positions P .. P+W-1       */
  int32_t chunk;         /* S, tokens per chunk; the library supports 8              */
  int32_t n_heads_q;     /* Hq, a multiple of n_heads_kv, Hq/Hkv <= 16               */
  int32_t n_heads_kv;    /* 1 <= Hkv <= 65535                                        */
  int32_t head_dim;      /* d; the library supports 128                              */
  int32_t rank;          /* r, coefficients per token; 64, 128, 256 or 512           */
  int32_t mlp_hidden;    /* H, value-MLP width; the library supports 256             */
  int32_t topk;          /* k >= 1 chunks kept per KV head (all if fewer candidates) */
  int32_t n_resid;       /* nR >= 0 stored residual rows per (sequence, KV head)     */
  int32_t n_cand;        /* candidates per (sequence, KV head): P/S without eviction,
                            the survivor count with cand_ids                          */
  int32_t coeff_fmt;     /* LOWRAM_FMT_* of coeff                                    */
  int32_t resid_fmt;     /* LOWRAM_FMT_* of res_val                                  */
  float rope_theta;      /* RoPE base; rotate-half pairing (i, i + d/2),
                            angle = position * theta^(-2i/d)                          */
  float softmax_scale;   /* logit scale, usually 1/sqrt(d)                           */
  /* Capacities, for caches that grow in place (lowram_append_*); 0 = dense.
     prefix_cap: coefficient rows per sequence, and (prefix_cap / S) landmark
     and descriptor rows per (sequence, KV head); >= prefix_len, a multiple
     of S.  window_cap: window rows per (sequence, KV head); >= window.  With
     cand_ids (eviction) both must be 0.  n_resid is the residual-row stride
     per (sequence, KV head); rows are reached through the descriptors only. */
  int32_t prefix_cap;
  int32_t window_cap;
} lowram_shape;

/* One layer's compressed cache (all device pointers). */
/* Layouts below are written for a dense cache; with capacities, P reads
   prefix_cap, P/S reads prefix_cap/S and W reads window_cap. */
typedef struct lowram_layer_cache {
  const void* coeff;            /* bf16: [NB][P][r];  int4: [NB][P][r/2] bytes                */
  const uint16_t* coeff_scale;  /* int4 only: [NB][P][r/32] fp16; NULL for bf16               */
  const uint16_t* basis;        /* [NB][Hkv][d][r] bf16: this layer's block of the group
                                   basis, transposed (basis[i][m] = B[m][col(layer,head,i)])  */
  const uint16_t* landmark;     /* [NB][Hkv][n_cand][d] bf16, mean post-RoPE key per chunk     */
  const int32_t* cand_ids;      /* [NB][Hkv][n_cand] ascending chunk ids of the candidates
                                   (eviction survivors), or NULL = every chunk 0..P/S-1       */
  const uint16_t* w1;           /* [NB][Hkv][H][d] bf16 value-MLP layer 1 weight              */
  const uint16_t* b1;           /* [NB][Hkv][H]    bf16                                        */
  const uint16_t* w2;           /* [NB][Hkv][d][H] bf16 layer 2 weight                        */
  const uint16_t* b2;           /* [NB][Hkv][d]    bf16                                        */
  const int32_t* res_idx;       /* [NB][Hkv][nR] ascending token ids (< P) with a residual    */
  const void* res_val;          /* bf16: [NB][Hkv][nR][d];  int4: [NB][Hkv][nR][d/2] bytes    */
  const uint16_t* res_scale;    /* int4 only: [NB][Hkv][nR][d/32] fp16; NULL for bf16         */
  const uint32_t* res_chunk_desc; /* [NB][Hkv][P/S] residual descriptor of chunk c: bits
                                   8..31 = row of res_idx holding the chunk's first residual
                                   token, bit i (< 8) set iff token c*S + i has a residual
                                   (see lowram_resid_chunk_desc)                              */
  const uint16_t* win_k;        /* [NB][Hkv][W][d] bf16 post-RoPE keys of the window          */
  const uint16_t* win_v;        /* [NB][Hkv][W][d] bf16 values of the window                  */
} lowram_layer_cache;

int lowram_abi_version(void);
const char* lowram_strerror(int status);

/* Bytes of device workspace lowram_decode_step needs for `shape` (a pure
   function of the shape; no HIP call). */
int lowram_workspace_bytes(const lowram_shape* shape, size_t* bytes);

/*
 * One decode step of one layer.
 *   q        [NB][Hq][d] bf16 post-RoPE queries; query head j uses KV head
 *            j / (Hq/Hkv) (GQA, LowRAM review, motivation paragraph).
 *   out      [NB][Hq][d] bf16 attention output (written).
 *   sel_out  optional [NB][Hkv][k] int32: the selected chunk ids, ascending,
 *            padded with -1 when fewer than k candidates exist; may be NULL.
 *   workspace / ws_bytes: device scratch of at least lowram_workspace_bytes.
 * Score of a candidate chunk c for KV head h: max over h's query heads j of
 * q_j . landmark[c] (raw dot product); the k largest are kept, exact ties
 * going to the lower chunk id.
 * The selected chunks run on one of two attention kernels: a persistent
 * producer/consumer kernel (one workgroup per CU working through groups of
 * 128-token tiles; fp16 RoPE, QK and GELU operands) once the problem gives
 * every CU at least two tiles, else a 4-wave kernel (bf16 operands).  The
 * environment variable LOWRAM_ATTEND=pipe or =wave, read at each call,
 * overrides the choice; both meet the same accuracy bound.  LOWRAM_PIPE_CUS=n
 * (n >= 1) plans the producer/consumer kernel for n CUs instead of the
 * device's count (fewer, longer workgroups; a testing aid, same results).
 */
int lowram_decode_step(const lowram_shape* shape, const lowram_layer_cache* cache,
                       const uint16_t* q, uint16_t* out, int32_t* sel_out,
                       void* workspace, size_t ws_bytes, void* stream);

/*
 * lowram_decode_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace: its kernels use a fixed device array of
 * LOWRAM_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one per GPU,
 * whose address is looked up (hipGetSymbolAddress) at the first call on each
 * device.  It calls no hipMalloc, hipFree or allocating library routine; the
 * caller still passes q, out, sel_out and the cache, as for
 * lowram_decode_step, and gets the same results.
 *   Limit: shapes whose lowram_workspace_bytes exceeds the scratch size are
 *   refused with LOWRAM_ERR_SCRATCH before any HIP call (e.g. at 262144
 *   tokens, top-1024 chunks and rank 512, about 7.7 MB per sequence: up
 *   to 8 sequences).
 *   Every call on a GPU shares that GPU's scratch, which keeps the last
 *   call's contents (nothing in it needs to start at zero): calls that
 *   overlap on one GPU (different streams, or threads without ordering) race
 *   and must be serialised by the caller.
 * Other errors as lowram_decode_step; LOWRAM_ERR_HIP also when the scratch's
 * address cannot be looked up, LOWRAM_ERR_UNSUPPORTED on a device ordinal
 * of 64 or more.
 */
int lowram_decode_step_noalloc(const lowram_shape* shape, const lowram_layer_cache* cache,
                               const uint16_t* q, uint16_t* out, int32_t* sel_out, void* stream);

/*
 * How lowram_decode_step schedules the selected chunks for `shape` on a
 * device of n_cu CUs (a scheduling query, not an operation of the method;
 * pure host computation, no HIP call).  mode: 0 the library's own choice,
 * 1 producer/consumer kernel forced, 2 4-wave kernel forced (as
 * LOWRAM_ATTEND=pipe / =wave).
 *   kernel           0 no selected chunks, 1 producer/consumer, 2 4-wave
 *   workgroups       producer/consumer kernel: min(n_cu, groups) (else 0)
 *   tiles_per_group  128-token tiles per group (else 0)
 *   groups_per_head  groups per (sequence, KV head) (else 0)
 *   partial_slots    partial states per (sequence, KV head) the merge
 *                    combines, window tiles included
 *   reserved_slots   partial slots per (sequence, KV head) in the workspace
 *                    (lowram_workspace_bytes), >= partial_slots
 *   window_kernel    where the exact window's tiles run: 0 no window, 1 as
 *                    extra workgroups of the landmark-score launch (with the
 *                    producer/consumer kernel), 2 in a 4-wave kernel launch
 *                    (field added in ABI version 3)
 * Returns LOWRAM_ERR_NULL, the shape errors of lowram_workspace_bytes, or
 * LOWRAM_ERR_SHAPE for n_cu < 1 or a mode outside 0..2.
 */
typedef struct lowram_attend_plan {
  int32_t kernel, workgroups, tiles_per_group, groups_per_head, partial_slots, reserved_slots;
  int32_t window_kernel;
} lowram_attend_plan;
int lowram_decode_plan(const lowram_shape* shape, int n_cu, int mode, lowram_attend_plan* plan);

/*
 * lowram_decode_step that also writes its intermediate stages (for stage
 * parity checks).  Every stage pointer may be NULL.
 *   scores_out [NB][Hkv][n_cand] fp32 landmark scores
 *   kpre_out, kpost_out, vhat_out [NB][Hkv][k*S][d] fp32: rebuilt pre-RoPE
 *            keys, rotated keys, predicted values + residuals, rows in the
 *            order of sel_out's chunks (ascending), S rows per chunk.
 */
int lowram_decode_stages(const lowram_shape* shape, const lowram_layer_cache* cache,
                         const uint16_t* q, uint16_t* out, int32_t* sel_out,
                         float* scores_out, float* kpre_out, float* kpost_out,
                         float* vhat_out, void* workspace, size_t ws_bytes, void* stream);

/*
 * lowram_decode_step that also records five caller-created hipEvent_t
 * (passed as void*) on `stream` around its kernels, for measurement:
 *   events[0] before the landmark scoring, [1] after it, [2] after the top-k
 *   selection, [3] after the fused rebuild + attention, [4] after the merge.
 * `events` may be NULL (then it is lowram_decode_step).  The events are only
 * recorded, never waited on.
 */
int lowram_decode_step_events(const lowram_shape* shape, const lowram_layer_cache* cache,
                              const uint16_t* q, uint16_t* out, int32_t* sel_out,
                              void* workspace, size_t ws_bytes, void* stream,
                              void* const* events);

/*
 * Shared-prefix multi-query decode: shape->batch queries (each a full set of
 * Hq query heads) attend to ONE compressed context, e.g. many questions over
 * one long document (review, results and limitations paragraphs: one
 * test-time fit per context; explainer, "Why it matters").  Every array of
 * `cache` has the layout of lowram_layer_cache for NB = 1 and is read by all
 * queries (batch stride 0); q, out, sel_out and the workspace are per query
 * ([NB][...] with NB = shape->batch).  Each query selects its own top-k
 * chunks.  `events` as in lowram_decode_step_events (may be NULL).
 */
int lowram_decode_shared(const lowram_shape* shape, const lowram_layer_cache* cache,
                         const uint16_t* q, uint16_t* out, int32_t* sel_out, void* workspace,
                         size_t ws_bytes, void* stream, void* const* events);

/* Dense GQA decode over the full bf16 cache: the uncompressed baseline the
   LowRAM pages compare against (review, results paragraph). */
typedef struct dense_shape {
  int32_t batch, ctx_len, n_heads_q, n_heads_kv, head_dim;
  float softmax_scale;
} dense_shape;

typedef struct dense_layer_cache {
  const uint16_t* k;  /* [NB][Hkv][T][d] bf16 post-RoPE keys */
  const uint16_t* v;  /* [NB][Hkv][T][d] bf16 values         */
} dense_layer_cache;

int dense_workspace_bytes(const dense_shape* shape, size_t* bytes);
int dense_decode_step(const dense_shape* shape, const dense_layer_cache* cache,
                      const uint16_t* q, uint16_t* out, void* workspace, size_t ws_bytes,
                      void* stream);

/*
 * Cache-layout helper: the residual descriptors of n_lists ascending lists of
 * n_resid token ids each (res_idx [n_lists][n_resid], desc [n_lists][n_chunks]):
 * desc[l][c] = (number of entries of res_idx[l] below c*chunk) << 8
 *            | bitmask of the tokens c*chunk + i (i < chunk) present in res_idx[l].
 * Requires chunk <= 8 and n_resid < 2^24.
 */
int lowram_resid_chunk_desc(const int32_t* res_idx, int32_t n_lists, int32_t n_resid,
                            int32_t n_chunks, int32_t chunk, uint32_t* desc, void* stream);

/* ---------------------------------------------------------------------------
 * Cache builder (prefill side).  Writes the arrays lowram_decode_step reads,
 * from a layer group's exact keys and each layer's exact values, as the
 * LowRAM pages describe compression:
 *   - review (agihunt.info), key paragraph: coefficients of the pre-RoPE keys
 *     in the group's shared basis, chunked prefix, mean post-RoPE key per
 *     chunk as its landmark;
 *   - review, value paragraph, and explainer (cctest.ai), "How the method
 *     works" / "Residuals for difficult tokens": values predicted from the
 *     rebuilt keys by the per-head MLP, exact residuals kept for the tokens
 *     it predicts worst.
 * The basis and the MLP weights are inputs; fitting them is not done here.
 * Conventions as above (device pointers, caller-owned, stream-ordered, no
 * allocation, status codes).
 * ------------------------------------------------------------------------- */
typedef struct lowram_build_shape {
  int32_t batch;         /* NB >= 1 sequences                                          */
  int32_t ctx_len;       /* T >= 1 tokens of exact keys / values per sequence          */
  int32_t window;        /* W, 0 <= W <= T: tokens P .. T-1 stay exact, P = T - W      */
  int32_t chunk;         /* S; P must be a multiple of it; the library supports 8      */
  int32_t n_heads_kv;    /* Hkv >= 1                                                   */
  int32_t head_dim;      /* d; the library supports 128                                */
  int32_t rank;          /* r; 64, 128, 256 or 512 (int4 coefficients: 128 and up)     */
  int32_t group_layers;  /* G >= 1 layers sharing one basis; key width D = G * Hkv * d */
  int32_t mlp_hidden;    /* H; the library supports 256                                */
  int32_t n_resid;       /* nR, 0 <= nR <= P residual rows kept per (sequence, head)   */
  int32_t coeff_fmt;     /* LOWRAM_FMT_* of the coefficients written                   */
  int32_t resid_fmt;     /* LOWRAM_FMT_* of the residual rows written                  */
  float rope_theta;      /* RoPE base, as in lowram_shape                              */
  /* Output capacities for a cache that later grows in place (0 = dense):
     coefficient rows per sequence (and prefix_cap / S landmark and descriptor
     rows per head), window rows per head, residual rows per head; each >=
     the size it holds, prefix_cap a multiple of S.  Inputs stay dense. */
  int32_t prefix_cap;
  int32_t window_cap;
  int32_t resid_cap;
} lowram_build_shape;

/*
 * Coefficients of one layer group: C[b][t][m] = sum_j X[b][t][j] B[b][m][j]
 * for the prefix tokens t < P (fp32 accumulation of bf16 products), stored
 * in shape->coeff_fmt.  Shared by the G layers of the group.
 *   keys   [NB][T][D] bf16 exact pre-RoPE keys of the group; column
 *          (l * Hkv + h) * d + i belongs to layer l of the group, KV head h
 *   basis  [NB][r][D] bf16 the group's basis B (rows orthonormal)
 *   coeff  out: bf16 [NB][P][r], or int4 [NB][P][r/2] bytes
 *   coeff_scale  out: int4 only, [NB][P][r/32] fp16; may be NULL for bf16
 * Needs no workspace.
 */
int lowram_build_coeff(const lowram_build_shape* shape, const uint16_t* keys,
                       const uint16_t* basis, void* coeff, uint16_t* coeff_scale, void* stream);

/* Inputs and outputs of one layer's build (all device pointers). */
typedef struct lowram_layer_build {
  const uint16_t* keys;         /* in:  [NB][T][D] bf16, as for lowram_build_coeff           */
  const uint16_t* group_basis;  /* in:  [NB][r][D] bf16                                       */
  const void* coeff;            /* in:  the group's coefficients from lowram_build_coeff      */
  const uint16_t* coeff_scale;  /* in:  int4 only                                             */
  const uint16_t* values;       /* in:  [NB][Hkv][T][d] bf16 exact values of this layer       */
  const uint16_t* w1;           /* in:  value MLP, layouts of lowram_layer_cache              */
  const uint16_t* b1;
  const uint16_t* w2;
  const uint16_t* b2;
  uint16_t* basis;              /* out: [NB][Hkv][d][r] this layer's basis blocks, transposed */
  uint16_t* landmark;           /* out: [NB][Hkv][P/S][d] bf16 mean post-RoPE key per chunk   */
  int32_t* res_idx;             /* out: [NB][Hkv][nR] ascending token ids                     */
  void* res_val;                /* out: bf16 [NB][Hkv][nR][d] or int4 [..][nR][d/2] bytes     */
  uint16_t* res_scale;          /* out: int4 only, [NB][Hkv][nR][d/32] fp16                   */
  uint32_t* res_chunk_desc;     /* out: [NB][Hkv][P/S] residual descriptors                   */
  uint16_t* win_k;              /* out: [NB][Hkv][W][d] bf16 post-RoPE keys of the window     */
  uint16_t* win_v;              /* out: [NB][Hkv][W][d] bf16 values of the window             */
  float* res_thresh;            /* out, optional: [NB][Hkv] the nR-th largest ||R_t|| (0 when
                                   every token is kept, +inf when nR = 0), the threshold of
                                   lowram_append_layer                                        */
  int32_t* res_count;           /* out, optional: [NB][Hkv] residual rows in use (= nR)        */
} lowram_layer_build;

/* Workspace bytes lowram_build_layer needs (pure function of the shape):
   about NB * Hkv * P * (4 d + 4) bytes, the fp32 residual of every prefix
   token and its error key, plus the top-nR selection's histograms. */
int lowram_build_layer_workspace_bytes(const lowram_build_shape* shape, size_t* bytes);

/*
 * One layer of the cache, layer_in_group in [0, G):
 *   basis     the layer's columns of B, per KV head, transposed (exact copy)
 *   landmark  per chunk c: mean over its S keys of RoPE(x_t, t), bf16
 *   residuals R_t = v_t - MLP(K_pre_t), K_pre_t = C_t (as stored) x basis
 *             block, MLP(k) = W2 gelu(W1 k + b1) + b2 with the erf GELU, all
 *             evaluated to fp32 accuracy; the nR tokens of largest ||R_t||_2
 *             (ties to the lower token), ascending, their R rows stored in
 *             shape->resid_fmt, and the per-chunk descriptors of
 *             lowram_resid_chunk_desc
 *   window    RoPE(x_t, t) and v_t of t = P .. T-1
 * Landmarks are written for all P/S chunks; eviction (cand_ids) is applied
 * by the caller after the build.
 */
int lowram_build_layer(const lowram_build_shape* shape, int32_t layer_in_group,
                       const lowram_layer_build* io, void* workspace, size_t ws_bytes,
                       void* stream);

/*
 * lowram_build_layer that also records five caller-created hipEvent_t
 * (passed as void*) on `stream`, for measurement: events[0] before its
 * kernels, [1] after the basis blocks, landmarks and window, [2] after the
 * residual prediction, [3] after the residual top-nR selection, [4] after the
 * residual rows and descriptors are stored.  `events` may be NULL.  The events
 * are only recorded, never waited on.
 */
int lowram_build_layer_events(const lowram_build_shape* shape, int32_t layer_in_group,
                              const lowram_layer_build* io, void* workspace, size_t ws_bytes,
                              void* stream, void* const* events);

/* ---------------------------------------------------------------------------
 * Window rollover (incremental append).  As decoding proceeds, the oldest S
 * tokens of the exact window are compressed into a new prefix chunk: their
 * coefficients, a landmark, and a residual test against the threshold the
 * cache was built with (the review's limitations paragraph: long generation
 * needs the newly generated suffix compressed periodically).  The cache must
 * have capacities (lowram_shape.prefix_cap / window_cap, n_resid = residual
 * rows per head) with room for the chunk; eviction (cand_ids) is not
 * supported.  `shape` describes the cache BEFORE the call (prefix_len = P,
 * window = W >= S, P + S <= prefix_cap); afterwards the caller's shape is
 * prefix_len = P + S, window = W - S.
 * ------------------------------------------------------------------------- */

/* Coefficient rows P .. P+S-1 of one layer group: keys_new [NB][S][D] (the S
   tokens' pre-RoPE keys of the group, D = group_layers * Hkv * d), basis
   [NB][r][D]; written into coeff (+ coeff_scale) in the cache layout. */
int lowram_append_coeff(const lowram_shape* shape, int32_t group_layers, const uint16_t* keys_new,
                        const uint16_t* basis, void* coeff, uint16_t* coeff_scale, void* stream);

/* One layer's part of the rollover (run after lowram_append_coeff).  The
   written arrays are the same ones `cache` points to, passed writable. */
typedef struct lowram_layer_append {
  const uint16_t* keys_new;     /* in:  [NB][S][D] as for lowram_append_coeff                  */
  const float* res_thresh;      /* in:  [NB][Hkv] residual threshold (lowram_layer_build)      */
  int32_t* res_count;           /* in/out: [NB][Hkv] residual rows in use                      */
  int32_t* res_dropped;         /* in/out: [NB][Hkv] += tokens over the threshold that found no
                                   free residual row (their values are then predicted only)   */
  uint16_t* landmark;           /* out: row P/S of each head                                  */
  int32_t* res_idx;             /* out: appended rows                                         */
  void* res_val;
  uint16_t* res_scale;          /* int4 only                                                  */
  uint32_t* res_chunk_desc;     /* out: entry P/S of each head                                */
  uint16_t* win_k;              /* in/out: rows S .. W-1 move to 0 .. W-S-1                   */
  uint16_t* win_v;              /* in/out: rows 0 .. S-1 are the new chunk's values           */
} lowram_layer_append;

/*
 * For each (sequence, KV head): landmark P/S = mean of RoPE(x_t, t) over the S
 * tokens; R_t = v_t - MLP(C_t B_blk) with v_t the window's rows 0 .. S-1,
 * evaluated to fp32 accuracy; each token with ||R_t|| >= res_thresh takes the
 * next free residual row (ascending token order); descriptor P/S written;
 * window rows S .. W-1 moved to 0 .. W-S-1.  Reads cache->coeff (rows P ..
 * P+S-1 included), coeff_scale, basis and the MLP.
 */
int lowram_append_layer(const lowram_shape* shape, int32_t group_layers, int32_t layer_in_group,
                        const lowram_layer_cache* cache, const lowram_layer_append* io, void* stream);
/* ---------------------------------------------------------------------------
 * Basis fit.  The review's key paragraph: adjacent layers share one low-rank
 * basis of their pre-RoPE keys, and a randomised Cholesky-QR replaces the
 * exact SVD (a reported 4x speed-up with no quality loss).  For each
 * sequence: Y = X^T Omega over the P prefix tokens, orthonormalised by
 * Cholesky-QR twice (CholQR2), then `power` passes Y <- CholQR2(X^T (X Y));
 * basis = Y^T, orthonormal rows.
 * ------------------------------------------------------------------------- */
typedef struct lowram_fit_shape {
  int32_t batch;         /* NB >= 1                                                     */
  int32_t ctx_len;       /* T rows of keys per sequence                                 */
  int32_t prefix_len;    /* P <= T tokens fitted; a multiple of 64                      */
  int32_t group_dim;     /* D = G * Hkv * d; a multiple of 128                          */
  int32_t rank;          /* r: 64, 128, 256 or 512                                      */
  int32_t power;         /* power passes, 0 .. 4 (1 recommended)                        */
} lowram_fit_shape;

/* Workspace for lowram_fit_basis: about D * P * 2 + r * P * 2 bytes (the keys
   transposed, one power-pass product), reused across the batch. */
int lowram_fit_basis_workspace_bytes(const lowram_fit_shape* shape, size_t* bytes);

/*
 *   keys      [NB][T][D] bf16 pre-RoPE keys of the layer group (rows < P used)
 *   omega_t   [NB][r][P] bf16 Gaussian test matrix, transposed (an input, so
 *             the caller fixes the random draw)
 *   basis     out: [NB][r][D] bf16 orthonormal rows, the lowram_build_* basis
 *   status    out: [NB] int32, 0 = ok, 1 = a Cholesky pivot was not positive
 *             (rank-deficient sketch; the basis is then not orthonormal)
 */
int lowram_fit_basis(const lowram_fit_shape* shape, const uint16_t* keys, const uint16_t* omega_t,
                     uint16_t* basis, int32_t* status, void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LOWRAM_H */
