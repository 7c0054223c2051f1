/*
 * zg_attn.h -- C ABI of the MI355X (gfx950) hybrid attention core of ZGCM-1.
 *
 * The method (all pages describe "ZGCM-1: A Fully Open and Extremely Efficient Foundation Model for
 * Math and Agentic Search"; the zh-TW translation page, section 2.1 "Model overview" and Figure 3):
 * most layers are gated sliding-window attention with a 128-token window, every sixth layer is full
 * causal attention; GQA with 32 query heads and 8 key/value heads of dim 128; q and k get RMSNorm and
 * partial RoPE (rotary fraction 0.33); a local layer's output is multiplied elementwise by
 * sigmoid(g_proj(h)) before o_proj, a global layer's is not. Section 2.3 "KV cache analysis": local
 * layers cache a fixed 128-token window, global layers the whole sequence.
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers owned by the caller; the library never allocates, frees or
 *    synchronises. Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = null stream).
 *  - bf16 tensors hold IEEE bfloat16 bit patterns (uint16). Layouts are row-major, last dim fastest.
 *  - Every argument is validated on the host before any launch. A bad argument returns a non-zero
 *    zg_status, leaves all buffers untouched and sets a thread-local message (zg_last_error). No
 *    entry point aborts or lets a C++ exception escape.
 *  - ZG_ERR_HIP: a HIP call or kernel launch reported an error. Faults inside a kernel surface at the
 *    caller's next synchronisation, as with any asynchronous launch.
 *  - NaN/Inf in inputs propagate; the hot path does no value checks.
 *  - No mutable global state except the static scratch of zg_attn_decode_noalloc (see there):
 *    calls from several host threads are safe; calls that share output buffers or a workspace
 *    must be ordered by the caller.
 */
#ifndef ZG_ATTN_H
#define ZG_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ZG_OK = 0,
  ZG_ERR_NULL = 1,        /* a required pointer is NULL */
  ZG_ERR_SHAPE = 2,       /* a size is negative/zero where it must be positive, or inconsistent */
  ZG_ERR_UNSUPPORTED = 3, /* a valid configuration the library has no kernel for */
  ZG_ERR_WORKSPACE = 4,   /* workspace pointer NULL or smaller than the *_workspace_bytes query */
  ZG_ERR_HIP = 5          /* HIP runtime / launch error */
} zg_status;

/* One attention layer's configuration.
 * Readings where the pages are silent: RMSNorm is per head over head_dim (one weight vector for q,
 * one for k); RMSNorm precedes RoPE; rotate-half pairs (i, i + rot_dim/2) with
 * theta_i = rope_base^(-2i/rot_dim); positions are 0-based; softmax scale 1/sqrt(head_dim). */
typedef struct {
  int32_t n_q_heads;     /* Hq, e.g. 32 */
  int32_t n_kv_heads;    /* Hkv, e.g. 8; Hq/Hkv must be 1, 2, 4 or 8 (else UNSUPPORTED) */
  int32_t head_dim;      /* D; 128 only (else UNSUPPORTED) */
  int32_t window;        /* W > 0: query i sees keys j with i-W < j <= i; W == 0: full causal */
  int32_t gated;         /* 1: out *= sigmoid(gate) elementwise; 0: gate ignored (may be NULL) */
  int32_t rot_dim;       /* rotated dims, even, 0 <= rot_dim <= 64 (ZGCM-1: floor(0.33*128) = 42) */
  double rope_base;      /* e.g. 1e4, 1e6, 1e7; > 1 */
  float rms_eps;         /* RMSNorm epsilon, e.g. 1e-6; >= 0 */
  float softmax_scale;   /* <= 0 selects 1/sqrt(head_dim) */
} zg_attn_cfg;

/* Elements between consecutive tokens of q, k, v, gate and out (token t of sequence b starts at
 * base + (b*T + t) * stride). Passing NULL means packed: Hq*D for q/gate/out, Hkv*D for k/v. A
 * stride must be >= the packed one and a multiple of 8 (16-byte aligned rows). */
typedef struct {
  int64_t q, k, v, gate, out;
} zg_token_strides;

/* ---------------------------------------------------------------------------------------------
 * Prefill: out[b,t,h,:] = gate?(sigmoid(gate[b,t,h,:])) * sum_j softmax_j(q_hat.k_hat_j*scale) v[b,j,h/G,:]
 * over the key set of query t (window or full causal), with q_hat/k_hat = RoPE(RMSNorm(.)) at
 * position pos0 + t. (zh-TW translation, section 2.1 and Fig. 3: the gated SWA formula.)
 *   q, gate, out: [B, T, Hq, D] bf16;  k, v: [B, T, Hkv, D] bf16  (see zg_token_strides)
 *   q_norm_w, k_norm_w: fp32[D] device pointers, or NULL for weight 1.
 *   workspace: device scratch of at least zg_attn_prefill_workspace_bytes(cfg, B, T) bytes (it holds
 *   the normalised, rotated keys and 2 KB of work counters for the attention launch; contents on
 *   entry do not matter); may be NULL when that query returns 0.
 * Numerics: fp32 norm/RoPE/softmax/accumulation; q_hat, k_hat and the softmax weights are rounded to
 * bf16 at the matrix-core inputs; out is rounded to nearest-even bf16.
 * Errors: NULL -> ZG_ERR_NULL; B < 1, T < 1, pos0 < 0, bad strides -> ZG_ERR_SHAPE; head_dim != 128,
 * Hq/Hkv not in {1,2,4,8}, rot_dim odd or > 64 -> ZG_ERR_UNSUPPORTED; small workspace ->
 * ZG_ERR_WORKSPACE. */
size_t zg_attn_prefill_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T);

zg_status zg_attn_prefill(const zg_attn_cfg* cfg, int32_t B, int32_t T, int64_t pos0,
                          const void* q, const void* k, const void* v, const void* gate,
                          const float* q_norm_w, const float* k_norm_w,
                          const zg_token_strides* strides,
                          void* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Chunked prefill through the decode caches: the T new tokens of every sequence sit at positions
 * pos0 .. pos0+T-1, keys of earlier positions come from the caches, and the call leaves the new
 * tokens' normalised, rotated keys and values in the caches, so decode (or a further chunk) can
 * continue from pos0 + T. (zh-TW translation, section 2.3: local layers keep a fixed 128-token
 * window, global layers the whole sequence.) Every sequence continues at the same pos0.
 *   window W > 0 (ring): k_cache, v_cache [B, W, Hkv, D] bf16; position p in slot p % W. On entry
 *            the slots hold positions max(0, pos0-W) .. pos0-1 (others are not read); on return
 *            positions max(0, pos0+T-W) .. pos0+T-1. cache_stride is ignored.
 *   window 0 (linear): k_cache, v_cache [B, cache_stride, Hkv, D] bf16; rows 0 .. pos0-1 hold the
 *            earlier positions; rows pos0 .. pos0+T-1 are written; cache_stride >= pos0 + T.
 *   q, k, v, gate, out, strides, norm weights: as for zg_attn_prefill (out = the T new rows).
 * The result equals zg_attn_prefill over the whole sequence 0 .. pos0+T-1, rows pos0 .. pos0+T-1,
 * up to rounding; pos0 = 0 with any cache contents is the plain prefill plus the cache fill.
 *   workspace >= zg_attn_prefill_cached_workspace_bytes(cfg, B, T) (0 for linear caches: the
 *   attention reads the cache; rings stage their W-1 context rows and the new rows, K and V:
 *   2 (W-1+T) rows of Hkv*256 bytes per sequence, each area rounded up to 256 bytes).
 * Errors as for prefill; linear cache_stride < pos0 + T -> ZG_ERR_SHAPE; (context + T) rows of
 * more than 4 GiB per sequence -> ZG_ERR_UNSUPPORTED. */
size_t zg_attn_prefill_cached_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T);

zg_status zg_attn_prefill_cached(const zg_attn_cfg* cfg, int32_t B, int32_t T, int64_t pos0,
                                 const void* q, const void* k, const void* v, const void* gate,
                                 const float* q_norm_w, const float* k_norm_w,
                                 const zg_token_strides* strides, void* k_cache, void* v_cache,
                                 int64_t cache_stride, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Training: forward with row log-sum-exp, and the backward pass of one attention layer.
 * (zh-TW translation, section 2.2 and section 3.1 quote training throughput; the layer is the
 * section 2.1 / Fig. 3 forward above.) Restrictions of these entry points: n_q_heads = 4 *
 * n_kv_heads (ZGCM-1's 32 / 8), packed tensors (q, gate, out, dout, dq, dgate [B, T, Hq, 128];
 * k, v, dk, dv [B, T, Hkv, 128], all bf16), positions 0 .. T-1, norm weights 1 (no weight
 * gradients). Other head ratios -> ZG_ERR_UNSUPPORTED.
 *
 * zg_attn_forward_train: out as zg_attn_prefill, plus lse [B, T, Hq] fp32, the natural-log
 * log-sum-exp of each query row's scaled scores over its key set (what the backward recomputes the
 * softmax from). workspace >= zg_attn_forward_train_workspace_bytes(cfg, B, T) (the normalised,
 * rotated keys: B T Hkv 256 bytes, rounded up to 256, then 2 KB of work counters).
 *
 * zg_attn_backward: gradients of L = sum(dout * out) with respect to q, k, v and the gate logits
 * (dgate, written only when cfg->gated), given the forward's inputs, its out and lse:
 *   dO = dout * sigmoid(gate) (dout when ungated), dgate = dout * out * (1 - sigmoid(gate)),
 *   D = rowsum(dout * out), P = exp(scale q_hat . k_hat - lse), dS = P (dO . v - D),
 *   dv = P^T dO, dq_hat = scale dS k_hat, dk_hat = scale dS^T q_hat, and dq, dk through RoPE's
 *   transpose and RMSNorm's derivative. dq, dk, dv, dgate are overwritten (bf16).
 * Numerics: q_hat, k_hat, dO, P and dS are rounded to bf16 at the matrix-core inputs; sums and the
 * norm/RoPE derivatives are fp32.
 *   workspace >= zg_attn_backward_workspace_bytes(cfg, B, T) (bf16 q_hat, k_hat, dO and a 32-byte
 *   row per query for lse and D: about B T (544 Hq + 256 Hkv) bytes).
 * Errors: NULL -> ZG_ERR_NULL; B < 1, T < 1 -> ZG_ERR_SHAPE; unsupported head ratio, head_dim,
 * rot_dim, or T * Hq * 256 bytes >= 4 GiB -> ZG_ERR_UNSUPPORTED; small workspace ->
 * ZG_ERR_WORKSPACE. */
size_t zg_attn_forward_train_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T);

zg_status zg_attn_forward_train(const zg_attn_cfg* cfg, int32_t B, int32_t T, const void* q,
                                const void* k, const void* v, const void* gate, void* out,
                                float* lse, void* workspace, size_t workspace_bytes, void* stream);

size_t zg_attn_backward_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T);

zg_status zg_attn_backward(const zg_attn_cfg* cfg, int32_t B, int32_t T, const void* q,
                           const void* k, const void* v, const void* gate, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           void* dgate, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Decode: one new token per sequence, attending over a KV cache of normalised, rotated keys.
 * (zh-TW translation, section 2.3: local layers keep a fixed 128-token window, global layers keep
 * the whole sequence; decoding is memory-bandwidth bound.)
 *   seqlens: device int32[B]; seqlens[b] >= 1 is the number of positions AFTER appending, so the new
 *            token sits at pos = seqlens[b] - 1 and must be < max_seqlen.
 *   window W > 0 (ring): k_cache, v_cache are [B, W, Hkv, D] bf16; position p lives in slot p % W
 *            (cache_stride is ignored and may be 0).
 *   window 0 (linear):  k_cache, v_cache are [B, cache_stride, Hkv, D] bf16; position p in row p;
 *            cache_stride >= max_seqlen.
 *   q_new, gate, out: [B, Hq, D] bf16; k_new, v_new: [B, Hkv, D] bf16.
 * The call RMSNorms and rotates q_new and k_new at pos, writes k_hat_new and v_new into the cache
 * row of pos, then attends over positions max(0, pos-W+1)..pos (ring) or 0..pos (linear) and
 * applies the gate if cfg->gated. The result equals prefill row pos over the same keys.
 *   workspace >= zg_attn_decode_workspace_bytes(cfg, B, max_seqlen) (split-KV partials).
 * Errors as for prefill; max_seqlen < 1 or cache_stride < max_seqlen (linear) -> ZG_ERR_SHAPE;
 * more than 2^21 keys to attend over (linear max_seqlen > 2097152) -> ZG_ERR_UNSUPPORTED.
 * seqlens values are device data and are not validated by the host; the kernels skip a sequence
 * whose seqlens[b] is < 1, or > cache_stride for a linear cache (no cache write, its out rows
 * unspecified), so no access leaves the caches; values above max_seqlen are otherwise a caller
 * error with unspecified results. */
size_t zg_attn_decode_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int64_t max_seqlen);

zg_status zg_attn_decode(const zg_attn_cfg* cfg, int32_t B, int64_t cache_stride,
                         int64_t max_seqlen, const void* q_new, const void* k_new,
                         const void* v_new, const void* gate, const float* q_norm_w,
                         const float* k_norm_w, void* k_cache, void* v_cache,
                         const int32_t* seqlens, void* out, void* workspace,
                         size_t workspace_bytes, void* stream);

/* zg_attn_decode without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation). The
 * workspace lives in a static device array of 96 MiB (100,663,296 bytes) that the library holds on
 * each GPU it runs on until the process ends; its address is looked up once per device, on the
 * first call with that device current. The call allocates and frees nothing.
 *   Arguments, layouts, numerics and errors as zg_attn_decode; in addition, when
 *   zg_attn_decode_workspace_bytes(cfg, B, max_seqlen) exceeds 96 MiB -> ZG_ERR_UNSUPPORTED
 *   (e.g. B = 64 with 32 query heads fits up to 94,208 keys per sequence: 92 chunks of 1024).
 *   Nothing in the scratch needs to start at zero: every value a call reads there it has written
 *   earlier on its own stream.
 *   All calls on one GPU share its array: calls that may overlap in time on one GPU (different
 *   streams, or host threads without ordering) race on it and give undefined results; order them. */
zg_status zg_attn_decode_noalloc(const zg_attn_cfg* cfg, int32_t B, int64_t cache_stride,
                                 int64_t max_seqlen, const void* q_new, const void* k_new,
                                 const void* v_new, const void* gate, const float* q_norm_w,
                                 const float* k_norm_w, void* k_cache, void* v_cache,
                                 const int32_t* seqlens, void* out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Decode over E4M3 KV caches: the FP8 format of the pages' forward pass (zh-TW translation,
 * section 3.1, hyper-parameters: mixed FP8, E4M3 forward), here halving the cache bytes that bound
 * decode (section 2.3). E4M3 is the OCP 8-bit float with 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, largest finite 448.
 *   k_cache, v_cache: as for zg_attn_decode but one byte per element; an entry c stands for
 *            c * k_scale (keys) or c * v_scale (values). The new token's k_hat / k_scale and
 *            v_new / v_scale are rounded to nearest-even E4M3, saturating at +-448, and written to
 *            the row of pos. k_scale, v_scale: finite and > 0.
 *   Everything else as zg_attn_decode (same workspace size).
 * Errors as zg_attn_decode; a bad scale -> ZG_ERR_SHAPE. */
zg_status zg_attn_decode_fp8(const zg_attn_cfg* cfg, int32_t B, int64_t cache_stride,
                             int64_t max_seqlen, const void* q_new, const void* k_new,
                             const void* v_new, const void* gate, const float* q_norm_w,
                             const float* k_norm_w, void* k_cache, void* v_cache, float k_scale,
                             float v_scale, const int32_t* seqlens, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* bf16 -> E4M3 conversion of n elements (e.g. a bf16 cache into an E4M3 cache): dst[i] =
 * E4M3(src[i] / scale), nearest-even, saturating at +-448. n a multiple of 16, 16-byte aligned
 * device pointers, scale finite and > 0; asynchronous on the stream. */
zg_status zg_kv_to_fp8(const void* src_bf16, void* dst_e4m3, int64_t n, float scale, void* stream);

/* ---------------------------------------------------------------------------------------------
 * KV-cache bytes of an n_layers stack (pure host arithmetic; zh-TW translation, section 2.3):
 *   sum over layers l = 1..n_layers of  rows(l) * 2 * n_kv_heads * head_dim * elem_bytes * batch,
 *   rows(l) = seqlen if layer l is global (global_every > 0 && l % global_every == 0, or window <= 0)
 *             else min(seqlen, window).
 * ZGCM-1: zg_kv_bytes(32, 6, 8, 128, 128, 2, 1, 262144) = 5,382,864,896 (5.0 GiB) and
 *         zg_kv_bytes(32, 1, ...) = 34,359,738,368 (32.0 GiB).
 * Returns 0 and sets zg_last_error on negative arguments or uint64 overflow. */
uint64_t zg_kv_bytes(int32_t n_layers, int32_t global_every, int32_t n_kv_heads, int32_t head_dim,
                     int32_t window, int32_t elem_bytes, int64_t batch, int64_t seqlen);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* zg_last_error(void);

/* Benchmark infrastructure, not part of the attention path (the benchmark uses it for the
 * streaming-read reference it reports beside the decode and local-layer rates): reads `bytes` (a positive multiple of 16)
 * from the device buffer `src` with streaming non-temporal 16-byte loads over `n_blocks`
 * workgroups of 256 lanes and writes one word per wave to `sink` (device, >= 4 * n_blocks words;
 * its values are meaningless). Timing it gives the device's streaming-read bandwidth, the
 * reference beside the 8 TB/s specification for the memory-bound kernels. Errors: NULL ->
 * ZG_ERR_NULL; bad sizes or alignment -> ZG_ERR_SHAPE. */
zg_status zg_hbm_read_probe(const void* src, int64_t bytes, uint32_t* sink, int32_t n_blocks,
                            void* stream);

/* ---------------------------------------------------------------------------------------------
 * Building blocks of one Pre-LN attention layer with projections (zh-TW translation, section 2.1
 * and Fig. 3: a normalised hidden state h feeds parallel q/k/v/gate projections; o_proj follows;
 * section 3.1 names Pre-LN).
 *
 * zg_rmsnorm: y[r,:] = bf16( x[r,:] / sqrt(mean(x[r,:]^2) + eps) * (w ? w : 1) ).
 *   x: fp32 [rows, dim]; w: fp32 [dim] or NULL; y: bf16 [rows, dim]. dim % 8 == 0, dim <= 8192. */
zg_status zg_rmsnorm(int64_t rows, int32_t dim, const float* x, const float* w, float eps,
                     void* y_bf16, void* stream);

/* zg_gemm_bf16: Y = X * W^T with fp32 accumulation.
 *   X: bf16 [M, K] (row stride K); W: bf16 [N, K] (row stride K).
 *   If residual != NULL: residual[m, n] += Y[m, n] (fp32 [M, N], row stride N).
 *   If y != NULL:        y[m, n] = bf16(Y[m, n]) (bf16, row stride ldy >= N).
 *   At least one of residual / y must be non-NULL. K % 64 == 0, N % 8 == 0, M >= 1. */
zg_status zg_gemm_bf16(int64_t M, int32_t N, int32_t K, const void* x_bf16, const void* w_bf16,
                       float* residual, void* y_bf16, int64_t ldy, void* stream);

/* zg_attn_layer: one whole layer, x <- x + o_proj(attn(RMSNorm(x))) on B*T tokens of width
 * hidden = Hq*D, in place on the fp32 residual x [B, T, hidden].
 *   w_qkvg: bf16 [(Hq + 2*Hkv + (gated ? Hq : 0)) * D, hidden], rows ordered q, k, v, gate;
 *   w_o: bf16 [hidden, Hq*D]. The input RMSNorm has weight 1 and eps cfg->rms_eps.
 *   workspace >= zg_attn_layer_workspace_bytes(cfg, B, T). */
size_t zg_attn_layer_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T);

zg_status zg_attn_layer(const zg_attn_cfg* cfg, int32_t B, int32_t T, float* x,
                        const void* w_qkvg, const void* w_o, const float* q_norm_w,
                        const float* k_norm_w, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ---------------------------------------------------------------------------------------------
 * E4M3 projections (zh-TW translation, section 3.1: the model's matrix multiplications run in FP8
 * with the E4M3 format on the forward pass). An E4M3 row matrix [rows, dim] (OCP E4M3: 4 exponent
 * bits, bias 7, 3 mantissa bits, largest finite 448; one byte per element, row stride dim) comes
 * with one fp32 scale per row, and row r stands for decode(code[r, :]) * scale[r]. Quantizing a
 * row h: amax = max |h|; scale = amax / 448 and codes = E4M3(h * (448 / amax)), each factor an
 * fp32 division rounded once, the codes rounded to nearest-even from the fp32 product and
 * saturated at +-448; a row of zeros gets scale 1 and zero codes.
 *
 * zg_rmsnorm_fp8: E4M3 rows of h = (x[r,:] / sqrt(mean(x[r,:]^2) + eps)) * (w ? w : 1), h in fp32.
 *   x: fp32 [rows, dim]; w: fp32 [dim] or NULL; y: [rows, dim] E4M3; y_scale: fp32 [rows].
 * zg_quant_rows_fp8: E4M3 rows of the bf16 rows x (row stride ldx >= dim, ldx % 8 == 0).
 *   Both: dim % 16 == 0, 16 <= dim <= 8192, rows >= 1; pointers 16-byte aligned. */
zg_status zg_rmsnorm_fp8(int64_t rows, int32_t dim, const float* x, const float* w, float eps,
                         void* y_fp8, float* y_scale, void* stream);
zg_status zg_quant_rows_fp8(int64_t rows, int32_t dim, const void* x_bf16, int64_t ldx,
                            void* y_fp8, float* y_scale, void* stream);

/* zg_gemm_fp8: Y[m, n] = x_scale[m] * w_scale[n] * sum_k X[m, k] * W[n, k], fp32 accumulation
 * of the exact E4M3 products.
 *   X: E4M3 [M, K] with x_scale fp32 [M]; W: E4M3 [N, K] with w_scale fp32 [N].
 *   If residual != NULL: residual[m, n] += Y[m, n] (fp32 [M, N], row stride N).
 *   If y != NULL:        y[m, n] = bf16(Y[m, n]) (bf16, row stride ldy >= N).
 *   At least one of residual / y must be non-NULL. K % 128 == 0, N % 8 == 0, M >= 1. */
zg_status zg_gemm_fp8(int64_t M, int32_t N, int32_t K, const void* x_fp8, const float* x_scale,
                      const void* w_fp8, const float* w_scale, float* residual, void* y_bf16,
                      int64_t ldy, void* stream);

/* zg_attn_layer_fp8: zg_attn_layer with E4M3 projections: h = E4M3 rows of RMSNorm(x);
 * [q, k, v, gate] = bf16(h W_qkvg^T); the attention as zg_attn_prefill; its bf16 output a as E4M3
 * rows; x += a W_o^T (fp32).
 *   w_qkvg: E4M3 [(Hq + 2*Hkv + (gated ? Hq : 0)) * D, hidden] with s_qkvg fp32 [rows];
 *   w_o: E4M3 [hidden, Hq*D] with s_o fp32 [hidden] (zg_quant_rows_fp8 of the bf16 weights gives
 *   both). workspace >= zg_attn_layer_fp8_workspace_bytes(cfg, B, T). */
size_t zg_attn_layer_fp8_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T);

zg_status zg_attn_layer_fp8(const zg_attn_cfg* cfg, int32_t B, int32_t T, float* x,
                            const void* w_qkvg_fp8, const float* s_qkvg, const void* w_o_fp8,
                            const float* s_o, const float* q_norm_w, const float* k_norm_w,
                            void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZG_ATTN_H */
