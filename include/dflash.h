/*
 * dflash.h -- C ABI of the MI355X (gfx950) block-diffusion drafting hot path.
 *
 * The library drafts a whole block of masked future tokens in one forward
 * pass of a small draft model that is conditioned on the target model's own
 * hidden states, and verifies drafted blocks greedily against the target's
 * logits.  Sources (news/explainer pages about DFlash):
 *   [P1] "DFlash: how block diffusion boosts NVIDIA Blackwell throughput"
 *        (dothoosh.com), section "Block-diffusion architecture";
 *   [P2] "DFlash-2: z-lab boosts speculative-decoding throughput"
 *        (dothoosh.com), sections "DFlash-2 mechanisms" and
 *        "Architecture-upgrade details";
 *   [P3] "NVIDIA tests DFlash to cut LLM inference bottlenecks"
 *        (stechtimes.com), section "DFlash moves token drafting to parallel
 *        compute".
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the comment says "host".
 *  - The caller allocates and owns every buffer (weights, KV cache, context
 *    lengths, workspace, inputs, outputs); the library keeps raw pointers,
 *    which must stay valid until dflash_destroy.  The library allocates no
 *    device memory at all.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls are asynchronous and stream ordered; they perform no host
 *    synchronisation, no allocation and no memset, so a sequence of calls can
 *    be captured into a HIP graph.  dflash_check / dflash_stats /
 *    dflash_stage_time are the exceptions: they synchronise `stream`.
 *  - Matrices are row-major [out_features, in_features].  "S" below is the
 *    storage type chosen by dflash_config.dtype (float or bfloat16) for
 *    weights, gains, the KV cache and the target hidden states.  All matrix
 *    products run on the bf16 matrix cores with fp32 accumulation (fp32
 *    weights are rounded to bf16 on load).  The attention queries and the
 *    attention output entering the O projection are a pair of bf16 values
 *    (value = hi + lo, two products each); so are the MLP inputs and the
 *    attention probabilities below 128 draft rows (batch * block), and the
 *    Q/K/V input with fp32 storage.  The other inputs (the Q/K/V input with
 *    bf16 storage, the MLP inputs and probabilities from 128 rows on, the
 *    context K/V projection and the LM head) take plain bf16.  The residual
 *    stream and the softmax stay fp32.
 *  - Errors the host can see (null pointer, bad size, unsupported shape)
 *    return DFLASH_EINVAL / DFLASH_EUNSUPPORTED before anything is enqueued;
 *    dflash_last_error() then holds a message.  HIP launch failures return
 *    DFLASH_EHIP.  Errors only the device can see (a context that would
 *    overflow max_ctx, a token id out of range) set a sticky bit in the
 *    device error word and skip the affected sequence's writes (an
 *    out-of-range token is embedded as zeros instead), and are reported
 *    by dflash_check().  No C++ exception crosses this boundary.
 *  - One host thread drives a context at a time, and its calls must be
 *    ordered (one stream, or streams synchronised by the caller): the calls
 *    share the context's workspace.  Two contexts share no state.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dflash_ctx dflash_ctx; /* opaque, owned by the library */

typedef enum {
  DFLASH_OK = 0,
  DFLASH_EINVAL = -1,      /* bad argument (host-checked) */
  DFLASH_EUNSUPPORTED = -2, /* shape or dtype the library does not implement */
  DFLASH_EHIP = -3,        /* a HIP runtime call or kernel launch failed */
  DFLASH_EDEVICE = -4      /* dflash_check: the device error word is non-zero */
} dflash_status;

enum { DFLASH_DTYPE_F32 = 0, DFLASH_DTYPE_BF16 = 1 };

/* Format of the draft KV cache (dflash_config.kv_dtype). */
enum {
  DFLASH_KV_STORAGE = 0, /* the storage type S, like the weights */
  DFLASH_KV_INT8 = 1     /* 8-bit integers with one float scale per 32 values (below) */
};

/* Device error-word bits (sticky until dflash_clear_errors). */
enum {
  DFLASH_ERR_FUSE_OVERFLOW = 1u << 0,   /* ctx_len[b] + t_new > max_ctx in fuse_ctx */
  DFLASH_ERR_TOKEN_RANGE = 1u << 1,     /* block id outside [0, vocab) in draft_block */
  DFLASH_ERR_VERIFY_OVERFLOW = 1u << 2, /* ctx_len[b] + n_d + 1 > max_ctx in verify */
  DFLASH_ERR_DRAFT_OVERFLOW = 1u << 3   /* ctx_len[b] + block > max_ctx in draft_block */
};

/* Stages, for dflash_stage_time. */
enum {
  DFLASH_STAGE_FUSE_FC = 0,  /* concat -> fusion linear (+ row sums of squares) */
  DFLASH_STAGE_CTX_KV = 1,   /* RMSNorm -> all layers' K/V projection, RoPE, cache append */
  DFLASH_STAGE_VERIFY = 2,   /* target argmax, accepted prefix, commit */
  DFLASH_STAGE_EMBED = 3,    /* block embedding */
  DFLASH_STAGE_QKV = 4,      /* RMSNorm -> Q/K/V projection, RoPE */
  DFLASH_STAGE_ATTN = 5,     /* non-causal GQA attention over [context ; block] */
  DFLASH_STAGE_OPROJ = 6,    /* output projection + residual (+ local conv) */
  DFLASH_STAGE_GATEUP = 7,   /* RMSNorm -> gate/up projection, SiLU product */
  DFLASH_STAGE_DOWN = 8,     /* down projection + residual */
  DFLASH_STAGE_LMHEAD = 9,   /* final RMSNorm -> LM head with per-tile argmax (the LM-head kernel alone) */
  DFLASH_STAGE_LAYER_GEMM = 10, /* the weight-streaming main kernel of every layer product (Q/K/V, O,
                                   gate/up, down) alone, without its finish kernel; overlaps stages 4-8 */
  DFLASH_N_STAGES = 11
};

/* Draft model shape and limits.  Requirements (else DFLASH_EUNSUPPORTED):
 * hidden, ffn and n_q_heads*head_dim multiples of 128; head_dim 64 or 128;
 * n_q_heads a multiple of n_kv_heads; block * (n_q_heads / n_kv_heads) <= 128;
 * vocab a multiple of 64; 1 <= block <= 64; 1 <= n_layers <= 8;
 * 1 <= n_target_layers <= 8; conv_width 0 or 3 (3 needs block to divide 16). */
typedef struct {
  int32_t hidden;          /* H */
  int32_t n_q_heads;       /* Hq */
  int32_t n_kv_heads;      /* Hkv */
  int32_t head_dim;        /* D */
  int32_t n_layers;        /* L */
  int32_t ffn;             /* F (SwiGLU inner size) */
  int32_t vocab;           /* V (embedding rows and shared LM head rows) */
  int32_t block;           /* Bs: rows of one drafted block */
  int32_t n_target_layers; /* K: target layers fused into the context feature */
  int32_t max_batch;       /* largest batch any call will pass */
  int32_t max_ctx;         /* KV cache rows per sequence */
  int32_t max_fuse_rows;   /* largest t_new per dflash_fuse_ctx call */
  int32_t conv_width;      /* 0, or 3 for the DFlash-2 local convolution */
  int32_t dtype;           /* DFLASH_DTYPE_F32 or DFLASH_DTYPE_BF16 (storage "S") */
  float rms_eps;           /* RMSNorm epsilon (1e-6 in the synthetic drafts) */
  float rope_theta;        /* rotary base (1e6) */
  int32_t kv_dtype;        /* DFLASH_KV_STORAGE (0) or DFLASH_KV_INT8 */
} dflash_config;

/* Draft weights (device pointers of storage type S).  Per-layer entries are
 * HOST arrays of n_layers device pointers; the arrays are copied at create. */
typedef struct {
  const void* embed;   /* [V, H] block-token embedding */
  const void* w_fc;    /* [H, K*H] fusion linear; column block j multiplies target layer j */
  const void* g_fc;    /* [H] gain of the RMSNorm after the fusion linear */
  const void* g_final; /* [H] gain of the final RMSNorm */
  const void* w_lm;    /* [V, H] shared LM head */
  const void* const* w_q;    /* [Hq*D, H] */
  const void* const* w_k;    /* [Hkv*D, H] (also projects the context feature) */
  const void* const* w_v;    /* [Hkv*D, H] (also projects the context feature) */
  const void* const* w_o;    /* [H, Hq*D] */
  const void* const* w_gate; /* [F, H] */
  const void* const* w_up;   /* [F, H] */
  const void* const* w_down; /* [H, F] */
  const void* const* g_in;   /* [H] RMSNorm before attention */
  const void* const* g_post; /* [H] RMSNorm before the MLP */
  const void* const* conv;   /* [H, 3] taps for rows (i-1, i, i+1); NULL when conv_width == 0 */
} dflash_weights;

/* Bytes of device workspace dflash_create needs for this configuration
 * (0 on an invalid configuration).  The workspace must be 256-byte aligned. */
size_t dflash_workspace_bytes(const dflash_config* cfg);

/* Bytes of ONE layer's K (or V) cache buffer (0 on an invalid configuration).
 * [P2] "DFlash-2: z-lab boosts speculative-decoding throughput", Precision
 * cost: an 8-bit KV cache is measured against f16 there (acceptance
 * 78.06% -> 74.88%) without a definition; DFLASH_KV_INT8 stores every row of
 * a KV head as 8-bit integers q in [-127, 127] with one float32 scale s per
 * 32 consecutive values (s = max|x| / 127 of those values, q = x / s rounded
 * half to even; the value read back is q * s; a run of zeros has s = 0).
 * Layout of one buffer (256-byte aligned):
 *   DFLASH_KV_STORAGE: S [max_batch, max_ctx, Hkv, D];
 *   DFLASH_KV_INT8:    int8 q [max_batch, max_ctx, Hkv, D], then, at byte
 *                      offset round_up(max_batch*max_ctx*Hkv*D, 256),
 *                      float32 s [max_batch, max_ctx, Hkv, D/32].
 * Every K/V entry the attention reads (the context rows and the block's own
 * rows, staged in the cache) goes through this format. */
size_t dflash_kv_layer_bytes(const dflash_config* cfg);

/* Create a context.
 *  kv_k, kv_v: HOST arrays of n_layers device pointers, each the persistent
 *     draft KV cache of one layer, dflash_kv_layer_bytes(cfg) bytes laid out
 *     as described there ([max_batch, max_ctx, Hkv, D] of S by default).
 *     K entries are stored after the rotary embedding.  [P1] "Block-diffusion
 *     architecture", KV-cache-integration bullet: the projected context
 *     features live in the draft KV cache and persist across iterations.
 *  ctx_len: device int32[max_batch], committed context rows per sequence;
 *     read and advanced by the library, may be set by the caller between
 *     calls (stream ordered).
 *  workspace: device buffer of dflash_workspace_bytes(cfg) bytes.  It is
 *     cleared here with a synchronous memset and receives the RoPE cos/sin
 *     table and a bf16 copy of every projection matrix (w_fc, w_q/k/v/o,
 *     w_gate/up/down, w_lm) in the matrix cores' fragment order: the products
 *     stream that copy, one contiguous 1 KB block per 16 rows x 32 columns,
 *     rather than 16 separate row pieces (create is not capturable); it
 *     belongs to the context until dflash_destroy and must not be written by
 *     the caller.  The copy takes the values the pointers hold at create:
 *     after changing those matrices, call dflash_reload_weights.
 * On success *out receives the context. */
dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w,
                            void* const* kv_k, void* const* kv_v, int32_t* ctx_len,
                            void* workspace, size_t workspace_bytes, dflash_ctx** out);

/* Re-copy the projection matrices from the pointers given at create into the
 * workspace's tiled copy (stream ordered, capturable; for a caller that has
 * changed the weights in place).  Later calls on the stream use the new
 * values. */
dflash_status dflash_reload_weights(dflash_ctx* ctx, void* stream);

/* Fuse target hidden states into the context feature and inject it into
 * every layer's K/V.  [P1] "Block-diffusion architecture", feature-injection
 * and KV-cache-integration bullets.
 *  hidden: HOST array of K device pointers, each [batch, t_new, H] of S, in
 *     target-layer order; the feature is
 *       c = RMSNorm(concat_j(hidden_j) . W_fc^T) * g_fc      (fp32 result)
 *     and for every layer l and row i of sequence b, at position
 *     p = ctx_len[b] + i:  K_l[b][p] = RoPE(c . W_k^l^T, p),
 *     V_l[b][p] = c . W_v^l^T.
 *  commit = 0: the rows are speculative (dflash_verify commits n+1 of them);
 *  commit = 1: ctx_len[b] += t_new (prompt pre-fill).
 *  feat_dbg: nullable fp32 [batch, t_new, H] output of c, for testing.
 * A sequence with ctx_len[b] + t_new > max_ctx gets DFLASH_ERR_FUSE_OVERFLOW
 * and no writes.  batch == 0 or t_new == 0 is a no-op. */
dflash_status dflash_fuse_ctx(dflash_ctx* ctx, int32_t batch, const void* const* hidden,
                              int32_t t_new, int32_t commit, float* feat_dbg, void* stream);

/* Greedy lossless verification with commit / rollback.  [P3] "DFlash moves
 * token drafting to parallel compute": the target keeps the verification
 * pass, so its greedy output is unchanged.
 *  target_logits: fp32 [batch, n_d + 1, V]; row i predicts the position that
 *     draft token i proposes (row n_d only supplies the bonus token).
 *  draft_ids: int32, sequence b's drafts at draft_ids[b*draft_stride + i],
 *     i < n_d.
 *  Per sequence: g_i = argmax_v target_logits[b, i, v] (lowest index on exact
 *  ties, NaN never chosen, all-NaN row gives 0); n = number of leading i with
 *  draft == g_i; outputs n_accept[b] = n, bonus[b] = g_n,
 *  out_tokens[b*(n_d+1) + i] = g_i for i <= n and -1 after; then
 *  ctx_len[b] += n + 1 (rows written speculatively by the preceding
 *  dflash_fuse_ctx beyond that are rolled back: left in place, never read,
 *  overwritten later).  Device counters {steps += batch, accepted += sum n,
 *  drafted += batch * n_d} accumulate (dflash_stats).
 *  0 <= n_d <= 64.  batch == 0 is a no-op. */
dflash_status dflash_verify(dflash_ctx* ctx, int32_t batch, const float* target_logits,
                            const int32_t* draft_ids, int32_t draft_stride, int32_t n_d,
                            int32_t* n_accept, int32_t* bonus, int32_t* out_tokens, void* stream);

/* Greedy verification without a context, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same rule, kernels and outputs as
 * dflash_verify, but nothing needs creating first.  Its only scratch, the
 * (row, vocabulary chunk) argmax keys, lives in a library-owned static device
 * array of 65536 keys (512 KB per device, held until the process ends), so
 *     batch * (n_d + 1) * ceil(vocab / 8192) <= 65536
 * (batch 32 at n_d 16 and vocab 151936 needs 10336), else DFLASH_EINVAL.
 * The call allocates nothing.  Every call on a device shares that array:
 * calls that overlap on one device (two streams, two threads) race, so they
 * must be ordered.
 *  target_logits: fp32 [batch, n_d + 1, vocab], 16-byte aligned; vocab a
 *     positive multiple of 64.
 *  ctx_len: device int32[batch], advanced by n + 1 per sequence unless
 *     ctx_len[b] + n_d + 1 > max_ctx (then left as is and DFLASH_ERR_VERIFY_OVERFLOW
 *     is or-ed into *error_word).
 *  stats: nullable device uint64[3] {steps, accepted, drafted}, accumulated.
 *  error_word: nullable device uint32, sticky bits as in dflash_check.
 *  draft_ids, draft_stride, n_d, n_accept, bonus, out_tokens: as dflash_verify.
 *  batch == 0 is a no-op. */
dflash_status dflash_verify_static(int32_t batch, int32_t vocab, const float* target_logits,
                                   const int32_t* draft_ids, int32_t draft_stride, int32_t n_d,
                                   int32_t* ctx_len, int32_t max_ctx, int32_t* n_accept, int32_t* bonus,
                                   int32_t* out_tokens, uint64_t* stats, uint32_t* error_word, void* stream);

/* Verification when the target samples at temperature T > 0.  The pages
 * measure a sampling mode but give no rule ([P1] Real-world integration,
 * the thinking setting); the rule here is the standard lossless
 * speculative-sampling rule for a drafter whose proposal is one token: with
 * p_i = softmax(target_logits[b][i] / T), draft d_i is accepted while
 * u[b][i][0] < p_i(d_i) (an id outside the vocabulary never is); the token
 * emitted at the first rejected row n is drawn from p_n with d_n removed
 * (nothing is removed for an id outside the vocabulary), or
 * at row n_d (all accepted) from p_{n_d}, as the inverse CDF over the
 * vocabulary in index order at u[b][n][1].  Every emitted token then has the
 * target's sampling distribution.
 *  uniforms: device fp32 [batch, n_d+1, 2] in [0, 1), supplied by the caller
 *     (the library draws no random numbers).
 *  Everything else as dflash_verify: bonus[b] receives the drawn token,
 *  out_tokens[b] = [d_0 .. d_{n-1}, drawn, -1 ...], ctx_len[b] += n + 1 and
 *  the counters advance; ctx_len[b] + n_d + 1 > max_ctx sets
 *  DFLASH_ERR_VERIFY_OVERFLOW and commits nothing.
 *  A NaN logit carries no mass (read as -inf): a draft there is rejected
 *  and no draw lands on it.  Each row needs a finite logit; +inf logits are
 *  outside this definition.
 *  temperature must be finite and > 0 with a finite 1/T (a subnormal T is
 *  rejected), else DFLASH_EINVAL and nothing is launched (T = 0 is
 *  dflash_verify). */
dflash_status dflash_verify_sample(dflash_ctx* ctx, int32_t batch, const float* target_logits,
                                   const int32_t* draft_ids, int32_t draft_stride, int32_t n_d,
                                   float temperature, const float* uniforms, int32_t* n_accept,
                                   int32_t* bonus, int32_t* out_tokens, void* stream);

/* Draft one block per sequence in a single forward pass.  [P1]
 * "Block-diffusion architecture": a whole block of masked future tokens per
 * pass; [P2] "DFlash-2 mechanisms": non-causal drafter; [P2]
 * "Architecture-upgrade details": local convolution between attention and MLP.
 *  block_ids: int32 [batch, Bs]; row i of sequence b sits at position
 *     ctx_len[b] + i.  The layer is pre-norm:
 *       u = RMSNorm(x) g_in; q,k,v = u W^T with RoPE on q,k;
 *       x += Attn(q, [K_l[b][0..ctx_len) ; k], [V_l ; v]) W_o^T   (no mask, GQA)
 *       x += conv3(x)                       (conv_width == 3 only)
 *       u = RMSNorm(x) g_post; x += (SiLU(u W_gate^T) * (u W_up^T)) W_down^T
 *     then draft_ids[b*Bs + i] = argmax_v (RMSNorm(x) g_final . W_lm^T)
 *     with the tie / NaN rule of dflash_verify.
 *  logits_dbg: nullable fp32 [batch, Bs, V]; hidden_dbg: nullable fp32
 *  [batch, Bs, H] final residual stream before the final norm (testing).
 *  Every layer's block K/V rows are staged in that layer's cache at rows
 *  ctx_len[b] + i (past the committed context: rows no committed state
 *  lives in, which the next dflash_fuse_ctx overwrites); a sequence with
 *  ctx_len[b] + Bs > max_ctx stages nothing, sets DFLASH_ERR_DRAFT_OVERFLOW
 *  and gets unspecified drafts.
 *  A block id outside [0, V) sets DFLASH_ERR_TOKEN_RANGE and embeds zeros.
 *  batch == 0 is a no-op. */
dflash_status dflash_draft_block(dflash_ctx* ctx, int32_t batch, const int32_t* block_ids,
                                 int32_t* draft_ids, float* logits_dbg, float* hidden_dbg,
                                 void* stream);

/* Synchronise `stream` and return the device error word in *error_bits (host).
 * Returns DFLASH_EDEVICE when it is non-zero, DFLASH_OK otherwise. */
dflash_status dflash_check(dflash_ctx* ctx, uint32_t* error_bits, void* stream);

/* Clear the device error word (stream ordered; uses a kernel, not a memset). */
dflash_status dflash_clear_errors(dflash_ctx* ctx, void* stream);

/* Synchronise `stream` and copy the verify counters to out3 (host):
 * {steps, accepted, drafted}.  Mean committed tokens per step =
 * 1 + accepted / steps; acceptance rate = accepted / drafted. */
dflash_status dflash_stats(dflash_ctx* ctx, uint64_t out3[3], void* stream);

/* Stage timing for profiling.  dflash_stage_timing(ctx, stage, 1) makes
 * later calls bracket every launch of that stage with HIP events (a host
 * pool of up to 4096 pairs, created here; no device memory); enable = 0 stops
 * recording.  dflash_stage_time synchronises `stream` and returns the mean
 * launch duration in milliseconds and the number of launches recorded, then
 * empties the pool. */
dflash_status dflash_stage_timing(dflash_ctx* ctx, int32_t stage, int32_t enable);
dflash_status dflash_stage_time(dflash_ctx* ctx, int32_t stage, double* mean_ms, int64_t* count,
                                void* stream);

/* Free the context (never the caller's buffers). NULL is a no-op. */
void dflash_destroy(dflash_ctx* ctx);

/* Message of the last non-OK status returned on this thread ("" if none). */
const char* dflash_last_error(void);

/* Version string of the library. */
const char* dflash_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
