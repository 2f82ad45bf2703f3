/*
 * qwm.h -- C ABI of a QuantWM 2-bit KV-cache library for AMD Instinct MI355X
 * (gfx950, CDNA4).
 *
 * The method is QuantWM ("QuantWM: Temporally Consistent 2-Bit KV Cache
 * Quantization for Video World Models", arXiv 2609.26425), known here through
 * the pages that report it:
 *   [digest]   "Flickering after quantization? A temporally stable 2-bit KV
 *              Cache compression framework for video world models emerges"
 *              (English news digest; paragraphs on QSAC, PSAC, the systems
 *              implementation and the attention analysis),
 *   [abstract] the Hugging Face Daily Papers abstract of the paper,
 *   [review]   "QuantWM: Temporally Consistent 2-Bit KV Cache Quantization for
 *              World Models and Video Generation" (summary; Eq. 7; FAQ).
 * A per-layer KV cache of already-generated frames grows with every frame
 * ([digest], opening paragraph).  Each cached Key is stored as a cluster
 * centre plus a 2-bit residual; the centre is chosen by QSAC, and the Key
 * error left after INT2 is compensated by PSAC along the principal directions
 * of historical Queries ([digest], QSAC and PSAC paragraphs).  Values take the
 * plain centre + 2-bit residual path.  Attention reconstructs the cache on the
 * fly ([digest], PSAC paragraph: compensation during cache reconstruction).
 *
 * Conventions
 *  - Every pointer is DEVICE memory unless its comment says "host".
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls that only enqueue work return as soon as it is enqueued; the ones
 *    marked "synchronous" wait for their stream before returning.
 *  - The caller owns every buffer (calibration block, cache block, workspace,
 *    inputs, outputs); the library never allocates device memory and keeps no
 *    pointer past a call except inside the caller-owned qwm_cache handle.
 *  - Activations are [heads][tokens][head_dim] tensors described by
 *    qwm_strides in ELEMENTS: element (h, t, j) sits at base +
 *    h*head + t*token + j.  The head_dim axis must be contiguous; the base
 *    pointer and token*element_size must be multiples of 16 bytes.
 *  - Errors are returned as negative status codes.  Every argument check runs
 *    on the host before anything is enqueued: on error nothing is launched and
 *    no cache counter moves.  Contents of device buffers are not inspected:
 *    inputs outside the binary16 range (|x| >= 65504) or non-finite inputs give
 *    unspecified values but never out-of-bounds accesses.
 *  - No call is re-entrant for one cache; one stream per cache.
 */
#ifndef QWM_H
#define QWM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QWM_ABI_VERSION 3

/* status codes */
#define QWM_OK 0
#define QWM_ERR_INVALID_ARG (-1)  /* null pointer, bad size, stride or alignment */
#define QWM_ERR_UNSUPPORTED (-2)  /* valid request outside what the kernels implement */
#define QWM_ERR_ALIGN (-3)        /* append of a token count that is not whole frames */
#define QWM_ERR_CAPACITY (-4)     /* append beyond max_frames, or workspace too small */
#define QWM_ERR_STATE (-5)        /* K/V counters disagree, or handle from another config */
#define QWM_ERR_HIP (-6)          /* a HIP runtime call failed; see qwm_status_string */

/* io_dtype */
#define QWM_BF16 0
#define QWM_F32 1

/* flags (ablation modes of the centre choice) */
#define QWM_UNIFORM_SENS 1u   /* QSAC distances and scores with s = 1 */
#define QWM_NO_RANGE_TERM 2u  /* choose argmin of the stage-1 distance (no INT2 score) */
#define QWM_QVG_MODE 3u       /* both: nearest Euclidean centre, the QVG baseline */
/* stage-2 score variants (ablations of the diagonal approximation, [review]
 * Eq. 7 and Table 10); they act only where stage 2 runs (K_c >= 2 without
 * QWM_NO_RANGE_TERM).  Both score the candidate's actual INT2 error
 * e = rho - Q(rho), Q quantizing each of the token's own 16-channel groups
 * with that group's own (zero, scale) (the tile arithmetic with a one-token
 * tile): */
#define QWM_EXACT_ERROR 4u     /* P = sum_j s_j e_j^2 (diagonal form) */
#define QWM_FULL_QUADRATIC 8u  /* P = e^T M e with the full Query second moment
                                  M (qwm_calib_import_moment); with
                                  QWM_UNIFORM_SENS, M = I.  Takes precedence
                                  over QWM_EXACT_ERROR. */

typedef struct qwm_config {
  int32_t abi_version;      /* QWM_ABI_VERSION */
  int32_t num_heads;        /* H >= 1 */
  int32_t head_dim;         /* d: 64 or 128 */
  int32_t frame_tokens;     /* F: tokens of one latent frame; appends are whole frames */
  int32_t max_frames;       /* cache capacity in frames */
  int32_t num_centroids_k;  /* C_K in [1, 512]: Key centres per head */
  int32_t num_centroids_v;  /* C_V in [1, 512]: Value centres per head */
  int32_t group_channels;   /* residual group width; must be 16 */
  int32_t group_tokens;     /* T in {1,2,4,8,16,32}: tokens sharing one (zero, scale) */
  int32_t top_candidates;   /* K_c in [0, 8]: QSAC stage-1 candidates (0: nearest) */
  int32_t rank;             /* r in [0, 32] (and <= d): PSAC principal directions */
  int32_t io_dtype;         /* QWM_BF16 or QWM_F32 for activations and centres */
  uint32_t flags;           /* QWM_UNIFORM_SENS | QWM_NO_RANGE_TERM | QWM_EXACT_ERROR |
                               QWM_FULL_QUADRATIC */
  int32_t reserved;         /* must be 0 */
} qwm_config;
/* Every call rejects with QWM_ERR_UNSUPPORTED a config whose append working
 * set does not fit one workgroup's 160 KiB of LDS: the larger codebook
 * (padded to a multiple of 64 centres, rows of d + 8 elements; twice that
 * for fp32 activations) plus fp64 U of the rank.  At d = 128 with bf16
 * activations, C = 512 runs up to r = 16 and r = 32 needs C <= 448. */

typedef struct qwm_strides {
  int64_t head;   /* elements between heads */
  int64_t token;  /* elements between tokens (>= head_dim) */
} qwm_strides;

/*
 * Byte sizes and offsets of the two caller-allocated blocks.
 *
 * Calibration block (per head h; all arrays [H][...] row-major):
 *   mu_k   [H][C_K][d]  centres of Keys, io dtype (bf16 / fp32)
 *   mu_v   [H][C_V][d]  centres of Values, io dtype
 *   sens   [H][d]       fp32 s = diag(M), the Query second moment's diagonal
 *   u      [H][d][r]    fp32 top-r eigenvectors of M (columns)
 *   derived, filled by qwm_calib_import / qwm_calibrate:
 *   u64    [H][d][RP]   fp64 copy of u (exact), rows padded with zeros to
 *                       RP = 8, 16 or 32 columns (the smallest >= r)
 *   sgroup [H][d/16]    fp64 S_g = sum of sens over group g
 *   norm_kw [H][C_K]    fp32 ||mu||_s^2 / 2 (sensitivity-weighted)
 *   norm_k  [H][C_K]    fp32 ||mu||^2 / 2
 *   norm_v  [H][C_V]    fp32 ||mu||^2 / 2
 *   head_max [H][4]     fp32 max_c ||mu_K||_s, max_c ||mu_K||, max_c ||mu_V||, 0
 *   mu_k16 [H][C_K][d]  fp16 copy of mu_k for the bf16 attention path; inside
 *                       each 16-channel group, position 2j holds channel j and
 *                       position 2j+1 channel j+8 (j = 0..7)
 *   mu_v16 [H][C_V][d]  the same for mu_v
 *   ut16   [H][UR][d]   fp16 U^T in the same channel order, UR = 16 (r <= 16)
 *                       or 32 rows; rows >= r are zero
 *   moment [H][d][d]    fp64 full Query second moment M (QWM_FULL_QUADRATIC
 *                       only, else 0 bytes; last in the block, written by
 *                       qwm_calib_import_moment and left alone by
 *                       qwm_calib_import)
 *
 * Cache block (capacity N = max_frames*F tokens, P = max_frames*ceil(F/T)
 * parameter tiles per head):
 *   idx_k    [H][N]        u8 if C_K <= 256 else u16: chosen Key centre
 *   codes_k  [H][N][d/16]  u32: 2-bit residual codes; word (t, g) holds the code
 *                          of channel 16g+i in bits [2i, 2i+1]
 *   params_k [H][P][d/16]  half2 (zero in the low half, scale in the high half)
 *                          of tile p = frame*ceil(F/T) + (t mod F)/T
 *   coef     [H][N][r]     int8 PSAC coefficients (absent when r = 0)
 *   coef_scale [H][N]      fp16 per-token coefficient scale (absent when r = 0)
 *   idx_v, codes_v, params_v  as above for Values.
 * Every array starts on a 256-byte boundary.
 */
typedef struct qwm_layout_info {
  uint64_t calib_bytes;
  uint64_t cache_bytes;
  uint64_t token_capacity;
  uint64_t tile_capacity;
  uint64_t mu_k, mu_v, sens, u, u64, sgroup, norm_kw, norm_k, norm_v, head_max, mu_k16, mu_v16, ut16, moment;
  uint64_t idx_k, codes_k, params_k, coef, coef_scale, idx_v, codes_v, params_v;
  uint32_t idx_k_bytes, idx_v_bytes;
} qwm_layout_info;

/* Host handle of one compressed cache.  Fill with qwm_cache_init.  The
 * caller owns it: lowering n_k and n_v together to a smaller whole number of
 * frames drops the newest frames (the next append overwrites them). */
typedef struct qwm_cache {
  void* base;          /* device, layout.cache_bytes */
  const void* calib;   /* device, layout.calib_bytes */
  int64_t n_k;         /* Keys appended so far (tokens) */
  int64_t n_v;         /* Values appended so far (tokens) */
  int32_t abi_version;
  int32_t reserved;
} qwm_cache;

int32_t qwm_abi_version(void);

/* Text for a status code (thread-local detail for QWM_ERR_HIP).  Never NULL. */
const char* qwm_status_string(int status);

/* Validates cfg and fills the block sizes and offsets (host out).  No HIP call. */
int qwm_layout(const qwm_config* cfg, qwm_layout_info* out);

/*
 * Compression accounting of n_tokens cached tokens ([digest], systems
 * paragraph; [review] FAQ: the ratio counts centres, quantization parameters
 * and compensation data).  stored_bytes (host out) counts the format's own
 * fields: indices, codes, tile parameters, INT8 coefficients and their scales,
 * the centres, U and s.  resident_bytes (host out, nullable) adds the derived
 * calibration fields and alignment that the library keeps resident.
 * original_bytes (host out) is 2*n_tokens*H*d*sizeof(io).  No HIP call.
 */
int qwm_footprint(const qwm_config* cfg, int64_t n_tokens, uint64_t* stored_bytes,
                  uint64_t* resident_bytes, uint64_t* original_bytes);

/*
 * Calibration on the host (all pointers host).  From historical Queries only
 * ([digest]: both designs use Query statistics of already-generated content;
 * [review] Eq. 7: E[(q^T e)^2] = e^T M e):
 *   M = (1/n_q) sum q q^T (uncentred, fp64); sens = diag(M);
 *   u = eigenvectors of the r largest eigenvalues of M, descending, each
 *       column's largest-magnitude entry positive (cyclic Jacobi, fp64);
 *   energy[h] = sum of the r largest eigenvalues / trace(M)
 *       ([digest], PSAC paragraph: top-8 directions hold about 71 %);
 *   mu_k, mu_v = Lloyd k-means of k_hist / v_hist (fp64, kmeans_iters rounds,
 *       Forgy start from a SplitMix64 partial Fisher-Yates shuffle seeded with
 *       seed + 2h for Keys and seed + 2h + 1 for Values, ties to the lowest
 *       index, empty clusters keep their centre), stored rounded to the io
 *       precision (bf16 round-to-nearest-even, or fp32).
 * Inputs are contiguous fp32 arrays [H][n][d] holding io-precision values;
 * outputs are fp32 arrays mu_k [H][C_K][d], mu_v [H][C_V][d], sens [H][d],
 * u [H][d][r], and energy fp64 [H] (nullable).  Requires n_kv >= max(C_K, C_V)
 * and n_q >= 1.  Deterministic; multi-threaded over heads.
 */
int qwm_calibrate_host(const qwm_config* cfg, const float* q_hist, int64_t n_q,
                       const float* k_hist, const float* v_hist, int64_t n_kv,
                       uint64_t seed, int32_t kmeans_iters, float* mu_k, float* mu_v,
                       float* sens, float* u, double* energy);

/*
 * Loads a calibration (host fp32 arrays in the shapes of qwm_calibrate_host's
 * outputs; mu values must be exact in the io precision) into the device
 * calibration block and computes its derived fields.  Synchronous on stream.
 */
int qwm_calib_import(const qwm_config* cfg, void* calib, const float* mu_k,
                     const float* mu_v, const float* sens, const float* u, void* stream);

/*
 * Loads the full Query second moment m (host fp64 [H][d][d], symmetric,
 * M = (1/n) sum q q^T per head, [review] Eq. 7) into the calibration block of
 * a QWM_FULL_QUADRATIC config (other configs: QWM_ERR_INVALID_ARG).
 * Synchronous on stream.
 */
int qwm_calib_import_moment(const qwm_config* cfg, void* calib, const double* m, void* stream);

/*
 * Device-side calibration: copies q_hist [H][n_q][d] and k_hist, v_hist
 * [H][n_kv][d] (io dtype, strided) to the host, runs qwm_calibrate_host and
 * qwm_calib_import (and, for QWM_FULL_QUADRATIC configs, imports
 * M = (1/n_q) sum q q^T of the same Queries).  energy (host, nullable)
 * receives [H] fp64.  Synchronous.
 */
int qwm_calibrate(const qwm_config* cfg, void* calib, const void* q_hist, int64_t n_q,
                  const qwm_strides* st_q, const void* k_hist, const void* v_hist,
                  int64_t n_kv, const qwm_strides* st_kv, uint64_t seed,
                  int32_t kmeans_iters, double* energy, void* stream);

/* Binds an empty cache (n_k = n_v = 0) to a cache block and a calibration
 * block.  No HIP call; appends overwrite every field they cover. */
int qwm_cache_init(const qwm_config* cfg, const void* calib, void* base, qwm_cache* cache);

/*
 * Quantize-append of n_new Keys (whole frames: n_new % F == 0, else
 * QWM_ERR_ALIGN; beyond capacity: QWM_ERR_CAPACITY) at token cache->n_k.
 * Per token ([digest] QSAC and PSAC paragraphs; [abstract]):
 *  QSAC stage 1: D_c = sum_j s_j (k_j - mu_cj)^2 over all C_K centres; keep
 *     the K_c smallest (ties to the lower index).
 *  QSAC stage 2: P_c = sum_g S_g range_g(rho)^2 with rho = fl32(k - mu_c) and
 *     range_g the max - min over the token's 16 channels of group g; choose
 *     argmin P (ties: smaller D, then lower index).  QWM_NO_RANGE_TERM or
 *     K_c = 0: argmin D.  QWM_UNIFORM_SENS: s = 1.  QWM_EXACT_ERROR and
 *     QWM_FULL_QUADRATIC replace P by the scores defined with those flags.
 *  INT2 per 16 channels x T tokens of one frame: z = fp16(min rho),
 *     s = fp16(fl32(fl32(max - min)/3)); code = #{i in 1..3 : rho >= fl32(z +
 *     (i - 1/2) s)}; s = 0 gives code 0.
 *  PSAC: e = k - (mu_c + fl32(z + code s)) in fp64; c = u^T e; c32 = fl32(c);
 *     sigma = fp16(fl32(max|c32|/127)); coef = clamp(rne(fl32(c32/sigma)),
 *     -127, 127) (0 when sigma = 0).
 * Decisions are exact up to score ties of relative size ~1e-15: stage 1 is an
 * MFMA screen whose error is bounded and whose ambiguous cases are rescored in
 * fp64; stage 2 and the projection run in fp64.  Advances cache->n_k after
 * enqueueing.  k_new is [H][n_new][d] in io dtype with strides st.
 */
int qwm_quantize_append_k(const qwm_config* cfg, qwm_cache* cache, const void* k_new,
                          int64_t n_new, const qwm_strides* st, void* stream);

/* Quantize-append of n_new Values: nearest Euclidean centre (ties to the
 * lower index) and INT2 residual tiles as for Keys, no compensation (the QVG
 * scheme the method builds on, [digest] QSAC paragraph).  Advances n_v. */
int qwm_quantize_append_v(const qwm_config* cfg, qwm_cache* cache, const void* v_new,
                          int64_t n_new, const qwm_strides* st, void* stream);

/* Both appends of the same n_new frames' tokens (Keys k_new with strides
 * st_k, Values v_new with st_v) in one launch: the same fields, bit for bit,
 * as qwm_quantize_append_k followed by qwm_quantize_append_v, with twice the
 * workgroups in flight.  Requires n_k == n_v (else QWM_ERR_STATE); checks both
 * inputs before launching anything.  Advances n_k and n_v. */
int qwm_quantize_append_kv(const qwm_config* cfg, qwm_cache* cache, const void* k_new,
                           const void* v_new, int64_t n_new, const qwm_strides* st_k,
                           const qwm_strides* st_v, void* stream);

/* Test and measurement hook: appends enqueued after this call add, with
 * device atomics, to counters (device uint32[4], nullable to stop; 4-byte
 * aligned): [0] Key tokens whose candidate set the append settled by exact
 * fp64 rescoring of the screen's uncertain band, [1] Key tokens that
 * searched all centres because the tracked list could not hold every
 * possible candidate, [2] and [3] the same for Values.  The pointer is a
 * process-wide setting read when each append is enqueued (graph-captured
 * appends keep the pointer they were captured with); set it from one thread
 * with no append in flight on another.  The caller clears the counters. */
int qwm_append_path_counters(void* counters);

/* Workspace bytes qwm_attention may use for n_q queries over n_tokens cached
 * tokens: partial results of query blocks whose key range is divided among
 * workgroups (bf16 activations: a fixed 2 x 256 slots of 256 rows, fp16, about
 * 34 MB at d = 128; fp32 activations: split-KV partials).  0 is always accepted by
 * qwm_attention (then every workgroup takes whole query blocks). */
size_t qwm_attention_workspace_size(const qwm_config* cfg, int64_t n_tokens, int64_t n_q);

/*
 * Attention of a query chunk q [H][n_q][d] (io dtype) over the compressed
 * cache (all n_k tokens visible; requires n_k == n_v, else QWM_ERR_STATE):
 *   k~_t = mu_K[idx_t] + rho_hat_t + u (coef_t * coef_scale_t)
 *   v~_t = mu_V[idx_t] + rho_hat^V_t
 *   l_t = scale * q.k~_t  (scale <= 0 selects 1/sqrt(d))
 *   out = sum_t softmax(l)_t v~_t  [H][n_q][d] io dtype (strides st_out)
 *   lse = log sum_t exp(l_t)       [H][n_q] fp32 (nullable)
 * ([abstract]: attention logits QK^T; [digest] PSAC paragraph; [review]: the
 * compensation is a low-rank correction of the logits).  Keys are rebuilt in
 * LDS as binary16 and the contractions run on fp16 MFMA with fp32
 * accumulation.  n_k = 0 gives out = 0 and lse = -inf.  workspace may be NULL
 * when ws_bytes = 0.
 */
int qwm_attention(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
                  const qwm_strides* st_q, float scale, void* out, const qwm_strides* st_out,
                  float* lse, void* workspace, size_t ws_bytes, void* stream);

/*
 * qwm_attention for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments (minus the workspace), results and
 * errors as qwm_attention with a workspace of QWM_NOALLOC_SCRATCH_BYTES; the
 * partial results go to a device array inside the library instead (32.5 MiB,
 * held on every GPU the library runs on until the process ends; enough for
 * the stream-K partials of bf16 activations at head_dim 128, else
 * QWM_ERR_CAPACITY).  No allocation happens in the call.  Every call on one
 * GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and give wrong results.  Nothing in the array needs
 * clearing: each partial result is written before it is read in the same call.
 */
#define QWM_NOALLOC_SCRATCH_BYTES 34078720u
int qwm_attention_noalloc(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
                          const qwm_strides* st_q, float scale, void* out, const qwm_strides* st_out,
                          float* lse, void* stream);

/* qwm_attention with two optional HIP events (hipEvent_t, NULL to skip)
 * recorded on stream immediately before and after the main attention kernel,
 * so that its duration can be measured apart from the pass that merges
 * partial results.  Same arguments, results and errors as qwm_attention. */
int qwm_attention_timed(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
                        const qwm_strides* st_q, float scale, void* out, const qwm_strides* st_out,
                        float* lse, void* workspace, size_t ws_bytes, void* stream,
                        void* ev_kernel_begin, void* ev_kernel_end);

/*
 * One generation step's attention: the query chunk attends to the compressed
 * cache and to the chunk's own uncompressed Keys and Values k_loc, v_loc
 * [H][n_loc][d] (bf16; strides st_k, st_v), all of them visible to every query
 * of the chunk.  The pages describe generation that reads the cached history
 * while the current frames are produced ([digest], opening paragraph: the
 * cache of historical frames grows as generation proceeds); the result is one
 * softmax over both key sets:
 *   out = sum_t softmax(l)_t w_t over t in (cache, local),
 *   l_t = scale q.k~_t (cache) or scale q.k_t (local), w_t = v~_t or v_t,
 *   lse = log sum_t exp(l_t).
 * It equals the log-sum-exp merge of qwm_attention over the cache with plain
 * softmax attention over the local keys.  Local rows enter the fp16
 * contraction like the queries (exact for |x| in [2^-17, 65504]).  bf16
 * activations only (fp32: QWM_ERR_UNSUPPORTED); n_loc = 0 is qwm_attention;
 * n_k = 0 (empty cache) is attention over the local chunk alone.  Workspace:
 * qwm_attention_workspace_size(cfg, n_k + n_loc, n_q).  Errors as for
 * qwm_attention, plus QWM_ERR_INVALID_ARG for misaligned local rows.
 */
int qwm_attention_local(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
                        const qwm_strides* st_q, const void* k_loc, const void* v_loc, int64_t n_loc,
                        const qwm_strides* st_k, const qwm_strides* st_v, float scale, void* out,
                        const qwm_strides* st_out, float* lse, void* workspace, size_t ws_bytes,
                        void* stream);

/*
 * Attention over a cache kept in calibration epochs.  The Query statistics
 * and centres come from content already generated ([digest], method
 * section: training-free, causal statistics of historical Queries); over a
 * long rollout ([digest] experiments paragraph: 1-minute generation) a caller
 * may calibrate again from recent frames and start a new cache block with the
 * new calibration for the frames that follow, so every stored frame keeps
 * the centres and U it was encoded with.  caches (host array, oldest first)
 * holds n_caches in [1, 64] such handles of the same cfg, each bound to its
 * own calibration block; their tokens, then the optional local chunk k_loc,
 * v_loc as in qwm_attention_local, form the key axis of one softmax:
 *   k~_t = mu_K^e[idx_t] + rho_hat_t + u^e (coef_t coef_scale_t) for a token
 *   t of epoch e (v~_t likewise with mu_V^e), out and lse as for
 *   qwm_attention_local.
 * One launch; U^T q is formed per epoch.  Every handle needs n_k == n_v (else
 * QWM_ERR_STATE); empty epochs are allowed.  n_caches > 64:
 * QWM_ERR_UNSUPPORTED; n_caches < 1 or caches NULL: QWM_ERR_INVALID_ARG.
 * bf16 activations only.  Workspace: qwm_attention_workspace_size(cfg,
 * total tokens, n_q).  With n_caches = 1 this is qwm_attention_local.
 */
int qwm_attention_epochs(const qwm_config* cfg, const qwm_cache* caches, int32_t n_caches, const void* q,
                         int64_t n_q, const qwm_strides* st_q, const void* k_loc, const void* v_loc, int64_t n_loc,
                         const qwm_strides* st_k, const qwm_strides* st_v, float scale, void* out,
                         const qwm_strides* st_out, float* lse, void* workspace, size_t ws_bytes, void* stream);

/* The logits l = scale q.k~ [H][n_q][n_k] fp32 (scale 1/sqrt(d) when <= 0),
 * exported by a debug variant of the attention kernel the activations' dtype
 * selects: the same tile rebuild and the same contraction S = Q' K~^T (for
 * bf16 activations: binary16 operands, fp32 accumulation), for logit parity
 * checks on small shapes ([abstract]: the logits Q K^T are the quantity the
 * method protects).  n_k = 0 or n_q = 0: nothing is written. */
int qwm_attention_logits(const qwm_config* cfg, const qwm_cache* cache, const void* q,
                         int64_t n_q, const qwm_strides* st_q, float scale, float* logits,
                         void* stream);

/*
 * Top-1 token selection ([digest], attention-analysis paragraph: the share of
 * queries whose highest-scoring historical token changes).  qwm_top1 writes
 * argmax_t q.k~_t over the compressed cache; qwm_dense_top1 writes argmax_t
 * q.k_t over original keys k [H][n_k][d] (io dtype).  Both: int32 [H][n_q],
 * ties to the lowest t.  qwm_top1 takes the scores S of the attention
 * kernel's top-1 variant (the rebuild and contraction of qwm_attention_logits);
 * qwm_dense_top1 takes fp32 dot products of the io values.
 */
int qwm_top1(const qwm_config* cfg, const qwm_cache* cache, const void* q, int64_t n_q,
             const qwm_strides* st_q, int32_t* top1, void* stream);
int qwm_dense_top1(const qwm_config* cfg, const void* q, int64_t n_q, const qwm_strides* st_q,
                   const void* k, int64_t n_k, const qwm_strides* st_k, int32_t* top1,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QWM_H */
