/*
 * tq_api.h - C ABI of the MI355X (gfx950) TurboQuant KV-cache hot path.
 *
 * The library stores new keys/values compressed into a paged KV cache and
 * runs decode attention straight from the compressed cache.  Sources of the
 * method (cited by page title and section):
 *   Roadmap : "From paper to practice: the TurboQuant integration roadmap of
 *             vLLM, SGLang and TRT-LLM" (miraclefarms notes, 2026-04-21)
 *   Hub     : "TurboQuant: extreme KV-cache compression for LLM inference"
 *             (pomoai hub page on the 0xSero/turboquant project)
 *   iThome  : the iThome article on TurboQuant KV-cache quantisation
 *             (article 10406003)
 *
 * Conventions for every entry point:
 *   - Return 0 (TQ_OK) on success or a negative TQ_E* code; no exception
 *     crosses the ABI.  tq_last_error() gives a thread-local message about
 *     the last failure on the calling thread.
 *   - Device pointers are plain HIP device addresses on the context's device;
 *     the caller owns every buffer it passes (inputs, pool, tables,
 *     workspace, outputs).  Quantise and decode never allocate or free.
 *   - Device work is enqueued asynchronously on the HIP stream passed as
 *     `stream` (a hipStream_t; NULL = the null stream); nothing synchronises.
 *     Errors found by host-side validation are reported before anything is
 *     enqueued.
 */
#ifndef TQ_API_H
#define TQ_API_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TQ_OK = 0,
  TQ_EINVAL = -1,       /* a bad argument (NULL, size, range, alignment) */
  TQ_EUNSUPPORTED = -2, /* a preset outside the supported set */
  TQ_EHIP = -3,         /* a HIP runtime call failed */
  TQ_ENOMEM = -4        /* host or device allocation failed (init only) */
};

enum { TQ_DTYPE_F32 = 0, TQ_DTYPE_BF16 = 1 };

/* Preset of one compressed cache.
 *   head_dim   : 128 or 256 (Hub, technical principle step 2: codebooks for
 *                head_dim 128 and 256).
 *   k_bits     : Lloyd-Max index bits per key coordinate, 2, 3 or 4 (Hub,
 *                step 2); each key coordinate also gets one QJL sign bit
 *                (Hub, step 3; Roadmap §1).  8 is accepted for MSE-only
 *                presets (the K8V4 preset of vLLM's path, iThome "which path
 *                vLLM takes"); 8-bit keys with the QJL sketch are rejected
 *                with TQ_EUNSUPPORTED, and tq_extend_attention does not take
 *                them.
 *   v_bits     : value bits, 2 or 4 (Hub, step 4).
 *   v_group    : value group size, must be 32 (Hub, step 4).
 *   block_size : tokens per paged block, must be 16.
 *   flags      : a bitwise or of
 *                TQ_PRESET_MSE_ONLY : keys without the QJL sketch (iThome,
 *                  "which path vLLM actually takes": presets with the
 *                  Hadamard rotation and MSE-quantised keys but no QJL): the
 *                  record then holds no sign bits and no residual norm, and
 *                  the score is n <q~, c[idx]> alone;
 *                TQ_PRESET_UNIFORM : equally spaced key centroids (Roadmap
 *                  §4.3, the "tq4u" mode: c_k = k step + c0) with the
 *                  least-squares step for the rotated-coordinate law
 *                  (tq_uniform_codebook) instead of the Lloyd-Max codebook;
 *                TQ_PRESET_ROTATE_V : values rotated with the keys' D2 H D1 /
 *                  sqrt(d) before their group quantisation (Roadmap §4.2,
 *                  W_O weight absorption): decode then returns rotated head
 *                  outputs, and tq_fold_output_projection gives the output
 *                  projection that undoes the rotation.
 *                Other bits are rejected with TQ_EUNSUPPORTED.
 *   seed       : seed of the library's own draw of D1, D2 and S when the
 *                caller does not pass them (splitmix64 counter stream; the
 *                signs are the top bit of consecutive outputs, the Gaussians
 *                come from Box-Muller on pairs of 53-bit uniforms). */
typedef struct {
  int32_t head_dim;
  int32_t k_bits;
  int32_t v_bits;
  int32_t v_group;
  int32_t block_size;
  int32_t flags;
  uint64_t seed;
} tq_preset;

enum { TQ_PRESET_MSE_ONLY = 1, TQ_PRESET_UNIFORM = 2, TQ_PRESET_ROTATE_V = 4 };

typedef struct tq_ctx tq_ctx; /* opaque; created by tq_codebook_init */

/* Byte offsets of the regions of one (block, KV head) record (all multiples
 * of 16).  With d = head_dim and 16 slots:
 *   kcodes [16][k_bits*d/8]  slot-major LSB-first Lloyd-Max index streams
 *   kqjl   [16][d/8]         slot-major QJL sign bits (1 = (S r)_i >= 0)
 *   kmeta  [16][2] fp16      (norm n, residual norm gamma) per slot
 *   vcodes [v_bits*d/32][16][4] dword w of every slot's value-code stream
 *                            together (byte f of slot s at ((f/4)*16+s)*4+f%4)
 *   vmeta  [d/32][16][2]     fp16 (scale, zero) per (group, slot)
 * MSE-only presets: kqjl is empty (kqjl == kmeta) and kmeta is [16] fp16 n. */
typedef struct {
  int64_t kcodes, kqjl, kmeta, vcodes, vmeta;
  int64_t record_bytes;
} tq_layout;

/* ------------------------------------------------------------------ init --
 * Solve the Lloyd-Max codebook of the rotated-coordinate law for
 * (head_dim, k_bits) in fp64 (Hub, technical principle steps 1-2: optimal
 * scalar codebooks for the Beta-distributed rotated coordinates; with
 * TQ_PRESET_UNIFORM the equally spaced codebook instead), round it to
 * fp32 centroids and fp32 midpoint thresholds, take the rotation signs and
 * the QJL matrix, and upload everything to the current HIP device.
 *   signs : [2][head_dim] int8, each +1 or -1 (row 0 = D1, row 1 = D2), or
 *           NULL to draw them from preset->seed (Roadmap §4.2: forward
 *           rotation D2 H D1).
 *   S     : [head_dim][head_dim] fp32 row-major QJL projection, or NULL to
 *           draw i.i.d. N(0, 1) from preset->seed (Hub, step 3: a d x d random
 *           projection).
 * Host pointers; copied.  *out receives a context owned by the caller, freed
 * by tq_ctx_destroy.  Not for the hot path (host work of a few ms). */
int tq_codebook_init(const tq_preset* preset, const int8_t* signs, const float* S, tq_ctx** out);

/* Free a context (device tables included).  NULL is accepted. */
int tq_ctx_destroy(tq_ctx* ctx);

/* Host copies of the context's tables, for tests.  Any output may be NULL.
 *   centroids [2^k_bits] fp32, thresholds [2^k_bits - 1] fp32,
 *   signs [2][head_dim] int8, S [head_dim][head_dim] fp32. */
int tq_ctx_tables(const tq_ctx* ctx, float* centroids, float* thresholds, int8_t* signs, float* S);

/* The preset a context was built with. */
int tq_ctx_preset(const tq_ctx* ctx, tq_preset* out);

/* Host-only helpers (no device needed). -----------------------------------
 * tq_lloyd_max: fp64 Lloyd-Max centroids [2^bits] (ascending) and thresholds
 * [2^bits - 1] for one coordinate of a uniform point on S^(head_dim-1);
 * head_dim >= 4 and even, bits 1..8.
 * tq_record_layout: region offsets of the paged record for a preset.
 * tq_draw_params: the seeded draw of D1, D2 (int8 [2][d]) and S (fp32 [d][d])
 * used when tq_codebook_init gets NULL arrays. */
int tq_lloyd_max(int32_t head_dim, int32_t bits, double* centroids, double* thresholds);
/* tq_uniform_codebook: the equally spaced codebook of least mean squared
 * error for the same law (centroids (k - (2^bits-1)/2) step, midpoint
 * thresholds), same argument rules as tq_lloyd_max. */
int tq_uniform_codebook(int32_t head_dim, int32_t bits, double* centroids, double* thresholds);
int tq_record_layout(const tq_preset* preset, tq_layout* out);
int tq_draw_params(uint64_t seed, int32_t head_dim, int8_t* signs, float* S);

/* Output projection with the inverse value rotation absorbed (Roadmap §4.2:
 * the inverse D1 H D2 / sqrt(d) -- the sign vectors in the reverse order of
 * the forward rotation -- folded into W_O once at load time, so decode over
 * a TQ_PRESET_ROTATE_V cache needs no inverse rotation):
 *   out[r][h d + j] = sum_i w_o[r][h d + i] Pi^-1[i][j],  h < num_q_heads,
 * i.e. every d-wide block of every row is mapped through D2 H D1 / sqrt(d)
 * (computed in fp64, rounded to fp32).
 *   signs : the context's [2][head_dim] int8 +-1 (row 0 = D1, row 1 = D2), as
 *           passed to tq_codebook_init or read back with tq_ctx_tables;
 *   w_o, out : host fp32 [rows][num_q_heads * head_dim] row-major; out may
 *           equal w_o.  Host-only; head_dim a power of two in 2..4096. */
int tq_fold_output_projection(int32_t head_dim, const int8_t* signs, const float* w_o, int64_t rows,
                              int32_t num_q_heads, float* out);

/* Bytes of one (block, KV head) record; 0 on a NULL context. */
size_t tq_block_bytes(const tq_ctx* ctx);

/* ----------------------------------------------------------- quantise ----
 * Compress num_tokens new keys and values of num_kv_heads heads each and
 * scatter them into the paged pool (Roadmap §3.1: rotation fused with the
 * quantiser in one launch; iThome "which path vLLM actually takes": quantise,
 * pack and write into the paged KV cache).  Per (token, head):
 *   n = ||k||; u = D2 (H/sqrt d) D1 k / n; idx_j = #{t : thr_t < u_j};
 *   r = u - c[idx]; gamma = ||r||; sign_i = [(S r)_i >= 0] (MSE-only presets
 *   stop at idx and store n alone);
 *   values (TQ_PRESET_ROTATE_V: first v <- fp32(D2 (H/sqrt d) D1 v), exact in
 *   fp64 before the one rounding) per group of 32: s = fp16((max-min)/(2^v_bits-1)), z = fp16(min),
 *   q = clamp(rint((v - z)/s), 0, 2^v_bits - 1) (q = 0 when s = 0).
 *   k, v         : device [num_tokens][num_kv_heads][head_dim], in_dtype
 *                  TQ_DTYPE_BF16 or TQ_DTYPE_F32; 16-byte aligned.
 *   slot_mapping : device int32 [num_tokens]; token i goes to block
 *                  slot_mapping[i] / 16, slot slot_mapping[i] % 16; a
 *                  negative entry skips the token.  Entries must be < 16 *
 *                  num_blocks and pairwise distinct (else the result is
 *                  undefined); they are not validated on the device.
 *   pool         : device [num_blocks][num_kv_heads][record_bytes], 16-byte
 *                  aligned; only the addressed slots are written.
 * num_tokens == 0 is a no-op. */
int tq_quantize_store(const tq_ctx* ctx, const void* k, const void* v, int32_t in_dtype, int64_t num_tokens,
                      int32_t num_kv_heads, const int32_t* slot_mapping, void* pool, int64_t num_blocks,
                      void* stream);

/* ------------------------------------------------------------- decode ----
 * Decode attention for one new query token per sequence, straight from the
 * compressed cache (Roadmap §3.2: rotate q once, score keys from the codes
 * through a per-query codebook table, exp2 online softmax, grouped query
 * heads; §3.1 and §7: a fixed split-KV grid and caller-owned workspace for
 * graph capture).  Score of query head h (KV head h / G) against cached
 * token t:
 *   est_t = n_t ( sum_j q~_j c[idx_tj] + sqrt(pi/2)/d gamma_t sum_i p_i (2 sign_ti - 1) ),
 *   q~ = D2 (H/sqrt d) D1 q, p = S q~, n_t and gamma_t the stored fp16 values
 *   (MSE-only presets: est_t = n_t sum_j q~_j c[idx_tj]);
 * recent full-precision tokens (Hub, vLLM integration: hybrid mode) score
 * <q, k> exactly.  out = softmax(sm_scale * scores) . values, values being
 * q s + z for cached tokens and the bf16 values for recent ones.  A sequence
 * with no tokens at all gets a zero output. */
typedef struct {
  const void* q;             /* device [batch][num_q_heads][head_dim], q_dtype */
  int32_t q_dtype;           /* TQ_DTYPE_BF16 or TQ_DTYPE_F32 */
  int32_t batch;             /* 0 .. 8192 */
  int32_t num_q_heads;
  int32_t num_kv_heads;      /* num_q_heads % num_kv_heads == 0, G <= 8; num_kv_heads x the
                                record bytes of a block < 2^31 */
  int32_t num_presets;       /* 1 or 2 */
  const tq_ctx* ctx[2];      /* same head_dim; one pool per preset */
  const void* pool[2];       /* device pools written by tq_quantize_store */
  int64_t pool_blocks[2];    /* blocks in each pool; tokens whose block id falls
                                outside [0, pool_blocks) are skipped */
  const int8_t* seq_preset;  /* device int8 [batch] in {0, 1}, or NULL = all 0 */
  const int32_t* block_tables; /* device int32 [batch][max_blocks_per_seq] */
  int32_t max_blocks_per_seq;
  const int32_t* seq_lens;   /* device int32 [batch]: cached tokens per sequence */
  const uint16_t* recent_k;  /* device bf16 [batch][num_kv_heads][recent_window][head_dim] or NULL */
  const uint16_t* recent_v;  /* same shape, NULL iff recent_k is NULL */
  const int32_t* recent_lens;/* device int32 [batch] in [0, recent_window], NULL iff recent_k is NULL */
  int32_t recent_window;
  float sm_scale;            /* <= 0 selects 1/sqrt(head_dim) */
  int32_t chunk_tokens;      /* tokens per split, a multiple of 32 in [32, 8192] (fixed at capture);
                                with no recent window and max_seq_len <= chunk_tokens each
                                sequence is a single split and the output is written by the
                                split launch itself (no separate combine launch) */
  int32_t max_seq_len;       /* largest seq_lens entry allowed (sizes the workspace) */
  void* workspace;           /* device, tq_decode_workspace_bytes(args) bytes, 256-byte aligned */
  size_t workspace_bytes;
  float* out;                /* device fp32 [batch][num_q_heads][head_dim] */
  float* scores_out;         /* device fp32 [batch][num_q_heads][scores_stride] or NULL:
                                raw scores, cached tokens first then recent ones */
  int32_t scores_stride;     /* >= max_seq_len + recent_window when scores_out != NULL */
  int32_t flags;             /* a bitwise or of TQ_DECODE_* below (0 = defaults) */
} tq_decode_args;

/* Decode flags.
 *   TQ_DECODE_DETERMINISTIC : accepted and has no further effect: every call
 *     takes the 32-token steps of a split in a fixed order per wave, so every
 *     fp32 sum is formed in the same order and the outputs (and scores) are
 *     bit-identical from run to run and between eager and graph-replayed
 *     launches, with or without the flag.
 * Other bits are rejected with TQ_EINVAL. */
enum { TQ_DECODE_DETERMINISTIC = 1 };

/* Workspace bytes the decode call needs for these arguments (only the shape
 * fields are read).  0 on invalid arguments. */
size_t tq_decode_workspace_bytes(const tq_decode_args* args);

/* Enqueue decode attention.  Device-side contents are clamped where a bad
 * value would address memory: seq_lens[b] is clamped to [0, max_seq_len],
 * recent_lens[b] to [0, recent_window], and a block id outside
 * [0, pool_blocks) skips its 16 tokens.  The launch configuration (LDS of the
 * recent window next to the kernel's own tables) is checked on the host:
 * a recent_window whose buffers do not fit a compute unit's 160 KB of LDS for
 * this head_dim and query-group size is rejected with TQ_EINVAL before
 * anything is enqueued. */
int tq_decode_attention(const tq_decode_args* args, void* stream);

/* ------------------------------------------------------------- extend ----
 * Extend (chunked prefill) attention: a chunk of new tokens per sequence
 * attends to that sequence's compressed prefix in the paged pool and,
 * causally, to the chunk itself (Roadmap §4.1: the fused extend kernel over
 * the compressed pool beside the fused decode kernel; §4.4: prefill is where
 * the rotation and quantisation cost shows).  Query token i of sequence b's
 * chunk sits at position prefix_lens[b] + i; its query head h (KV head
 * h / G) scores
 *   the prefix tokens t < prefix_lens[b] with the decode estimator
 *     est_t = n_t ( sum_j q~_j c[idx_tj] + sqrt(pi/2)/d gamma_t sum_i p_i (2 sign_ti - 1) )
 *     (MSE-only presets: the first term alone), values q s + z;
 *   the chunk tokens j <= i exactly, <q_i, k_j>, values v_j (bf16);
 * out = softmax(sm_scale * scores) . values.  The chunk's keys and values are
 * not read from the pool: store them with tq_quantize_store (before or after
 * this call; the order does not matter).
 *   q       : device bf16 [num_tokens][num_q_heads][head_dim], the chunks of
 *             all sequences one after another (rows cu_chunk[b] ..
 *             cu_chunk[b+1] - 1 for sequence b); 16-byte aligned.
 *   k, v    : device bf16 [num_tokens][num_kv_heads][head_dim], same rows.
 *   cu_chunk: device int32 [batch + 1], non-decreasing, cu_chunk[0] = 0;
 *             chunk lengths are clamped to max_chunk.
 *   prefix_lens : device int32 [batch]; clamped to [0, max_prefix_len].
 *   block_tables: device int32 [batch][max_blocks_per_seq]; block ids outside
 *             [0, pool_blocks) make their 16 prefix tokens drop out.
 *   out     : device fp32 [num_tokens][num_q_heads][head_dim].
 * Supported: head_dim 128 and query heads per KV head G in {1, 2, 4, 8}
 * (others: TQ_EUNSUPPORTED).  One launch, no workspace, no allocation. */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_chunk;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_chunk;          /* >= every chunk length; sizes the grid */
  const tq_ctx* ctx;
  const void* pool;
  int64_t pool_blocks;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* prefix_lens;
  int32_t max_prefix_len;     /* <= 16 * max_blocks_per_seq */
  float sm_scale;             /* <= 0 selects 1/sqrt(head_dim) */
  float* out;
} tq_extend_args;

int tq_extend_attention(const tq_extend_args* args, void* stream);

/* ------------------------------------------------- decode, no allocation --
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, validation and results as tq_decode_attention, except that
 * args->workspace and args->workspace_bytes are ignored: the split partials
 * go to a scratch array of TQ_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds in device memory (one per GPU, reserved with the library's code
 * object and kept until the process ends).  A call whose partials need more
 * than that (tq_decode_workspace_bytes(args) > TQ_NOALLOC_SCRATCH_BYTES) is
 * rejected with TQ_EINVAL before anything is enqueued.  Nothing is allocated,
 * freed or cleared: every partial is written before it is read.  Calls on one
 * GPU share its scratch array, so calls whose launches overlap (two streams,
 * or two host threads, on the same device) race and may corrupt each other's
 * outputs; serialise them on one stream. */
#define TQ_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int tq_decode_attention_noalloc(const tq_decode_args* args, void* stream);

/* Thread-local message of the last failure ("" if none). */
const char* tq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_API_H */
