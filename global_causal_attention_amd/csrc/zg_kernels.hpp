// Internal launch interface between the C ABI (api.cpp) and the gfx950 kernels (*.hip).
// Host-visible parameter blocks; all pointers are device pointers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zg {

constexpr int kMaxRotHalfHost = 32;

struct RopeTableH {
  double rev[kMaxRotHalfHost];  // theta_i / (2 pi) for i < half
  int32_t half;
};

// Normalise + rotate keys into a packed [B, T, Hkv, 128] bf16 buffer.
struct KPrepParams {
  const uint16_t* k;
  uint16_t* khat;
  const float* k_norm_w;
  int64_t sk;  // token stride of k (elements)
  int32_t B, T, Hkv;
  int64_t pos0;
  // output rows: k_hat of (b, t) goes to row out_row0 + t of sequence b, sequences out_rows
  // rows apart (out_rows = T, out_row0 = 0 for a packed [B, T, Hkv, 128] result)
  int64_t out_rows, out_row0;
  float eps;
  RopeTableH rope;
  // Folding for the banded streaming kernel: when set, dims < rot_dim are multiplied by
  // fold_scale and dims >= rot_dim by fold_scale * fold_w[d] (fold_w may be null: 1).
  int32_t fold;
  float fold_scale;
  const float* fold_w;
  // Ring write of a chunked prefill: when ring_k is non-null, rows t >= ring_t0 (the last
  // ring_w positions) also go to slot (pos0 + t) % ring_w of their sequence in the rings
  // [B, ring_w, Hkv, 128]: the unfolded k_hat to ring_k, and row t of ring_v_src (token stride
  // ring_sv) unchanged to ring_v.
  uint16_t* ring_k;
  uint16_t* ring_v;
  const uint16_t* ring_v_src;
  int64_t ring_sv;
  int32_t ring_w, ring_t0;
  // When non-null, the first launch block also zeroes these words (the item counters of the
  // prefill kernel that follows this launch on the stream).
  uint32_t* zero_words;
  int32_t n_zero_words;
};

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* khat;  // packed [B, T, Hkv, 128]
  const uint16_t* v;
  const uint16_t* gate;
  uint16_t* out;
  const float* q_norm_w;
  int64_t sq, sv, sg, so;  // token strides (elements)
  int32_t B, T, Hq, Hkv;
  int64_t pos0;
  int32_t window;
  int32_t n_qtiles;
  int32_t seg_steps;  // banded kernel: 64-query steps per workgroup
  int32_t persist;    // tiled kernel: one workgroup per CU walks the items (set by the launcher)
  // Keys: sequence b's k_hat and v rows start kv_rows rows apart; n_keys of them are valid, and
  // query row t is key row qoff + t (rows before qoff are earlier positions from a cache).
  // Plain prefill: kv_rows = n_keys = T, qoff = 0.
  int64_t kv_rows;
  int32_t n_keys, qoff;
  // optional [B, T, Hq] fp32: natural-log log-sum-exp of each query row's scaled scores (plain
  // prefill with qoff = 0; the backward pass recomputes the softmax from it)
  float* lse;
  float eps;
  float scale_log2;  // softmax scale * log2(e)
  RopeTableH rope;
  // Tiled kernel, persistent launch: kSchedWords words (zeroed before the launch) holding the item
  // counters of the dynamic schedule, kSchedStride words apart; null: the static item schedule.
  uint32_t* counters;
};

// Item counters of the persistent tiled kernel's dynamic schedule (a heavy and a light queue per
// XCD, a 128-byte line each): the bytes a caller's workspace reserves for them.
constexpr int kSchedStride = 32;
constexpr int kSchedWords = 16 * kSchedStride;
constexpr int kSchedBytes = kSchedWords * 4;

// Split-KV decode: keys per chunk (one workgroup each), and the most chunks one sequence may have.
constexpr int kDecodeChunkKeys = 1024;
constexpr int kDecodeMaxChunks = 2048;

struct DecodeParams {
  const uint16_t* q_new;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* gate;
  const float* q_norm_w;
  const float* k_norm_w;
  uint16_t* k_cache;
  uint16_t* v_cache;
  const int32_t* seqlens;
  uint16_t* out;
  float* qhat;      // workspace: [B, Hq, 128] fp32 (bf16-rounded values)
  float* partial;   // workspace: [B, Hq, n_chunks, 130] fp32 (m, l, o[128])
  int32_t B, Hq, Hkv;
  int32_t window;   // ring slots (0: linear)
  int64_t rows;     // rows per sequence in the cache (window or cache_stride)
  int32_t chunk;    // keys per split
  int32_t n_chunks; // max splits per sequence
  int32_t gated;
  float eps;
  float scale_log2;
  RopeTableH rope;
  // E4M3 caches (one byte per element) holding k_hat / k_scale and v / v_scale: the new row is
  // written as E4M3 of its value times k_inv / v_inv, and outputs are multiplied by v_scale
  // (k_scale is folded into scale_log2 by the host).
  int32_t fp8;
  float k_inv, v_inv, v_scale;
};

struct ToFp8Params {
  const uint16_t* src;  // bf16
  uint8_t* dst;         // E4M3
  int64_t n;            // elements, multiple of 16
  float inv_scale;
};
hipError_t launch_to_fp8(const ToFp8Params& p, hipStream_t s);

// Backward pass of one attention layer (4 query heads per KV head, head dim 128, packed
// [B, T, H, 128] tensors, positions 0 .. T-1, norm weights 1).
struct BwdParams {
  const uint16_t *q, *k, *v, *gate, *out, *dout;  // bf16 inputs (gate null when ungated)
  const float* lse;                              // [B, T, Hq] natural log, from the forward
  uint16_t *dq, *dk, *dv, *dgate;                // bf16 outputs (dgate null when ungated)
  // workspace
  uint16_t* qc;    // [B, T, Hq, 128] bf16(q_hat * scale * log2 e), as the forward's operand
  uint16_t* khat;  // [B, T, Hkv, 128] bf16(k_hat)
  uint16_t* dO;    // [B, T, Hq, 128] bf16(dout * sigmoid(gate)); dout itself when ungated
  uint16_t* aux;   // [B, T, Hq, 16] bf16: (-L log2 e, -D), each as three bf16 terms + zeros
  int32_t B, T, Hq, Hkv, window, gated;
  int32_t n_qtiles;
  int64_t pos0;
  float eps, scale;  // scale: the softmax scale (natural units)
  RopeTableH rope;
};
hipError_t launch_backward(const BwdParams& p, hipStream_t s);

struct RmsNormParams {
  const float* x;
  const float* w;
  uint16_t* y;
  int64_t rows;
  int32_t dim;
  float eps;
};

struct GemmParams {
  const uint16_t* x;  // [M, K]
  const uint16_t* w;  // [N, K]
  float* residual;    // [M, N] or null
  uint16_t* y;        // [M, ldy] or null
  int64_t ldy;
  int64_t M;
  int32_t N, K;
};

// E4M3 rows with one fp32 scale per row: row r stands for decode(code[r, :]) * scale[r].
// Quantization of a row h: scale = amax / 448, codes = E4M3(h * (448 / amax)) (both factors
// rounded to fp32 once); a row of zeros gets scale 1 and zero codes.
struct RmsNormFp8Params {   // y = E4M3 rows of RMSNorm(x) * w (x fp32)
  const float* x;
  const float* w;
  uint8_t* y;
  float* y_scale;
  int64_t rows;
  int32_t dim;
  float eps;
};
struct QuantRowsParams {    // y = E4M3 rows of x (bf16, row stride ldx)
  const uint16_t* x;
  int64_t ldx;
  uint8_t* y;
  float* y_scale;
  int64_t rows;
  int32_t dim;
};
struct GemmFp8Params {      // Y[m, n] = x_scale[m] w_scale[n] sum_k X[m, k] W[n, k]
  const uint8_t* x;   // [M, K] E4M3
  const float* x_scale;
  const uint8_t* w;   // [N, K] E4M3
  const float* w_scale;
  float* residual;    // [M, N] or null: += Y
  uint16_t* y;        // [M, ldy] or null: bf16(Y)
  int64_t ldy;
  int64_t M;
  int32_t N, K;
};

// Row copies between token-major [B, rows, Hkv, 128] buffers (caches, staging): row j of
// sequence b goes from src row src_row0 + j to dst row dst_row0 + j; a side whose ring > 0 takes
// its row index modulo ring (a ring cache's slot).
struct RowCopyParams {
  const uint16_t* src;
  uint16_t* dst;
  int64_t src_bstride, dst_bstride;  // rows per sequence
  int64_t src_row0, dst_row0;
  int64_t src_stride, dst_stride;    // elements per row (token stride)
  int64_t src_ring, dst_ring;
  int32_t row_elems;                 // elements copied per row (multiple of 8)
  int32_t rows;                      // rows per sequence
  int32_t B;
  // When fold is set, element e of a row is multiplied as KPrepParams::fold does for head dim
  // e mod 128 (fold_scale, times fold_w for dims >= rot_dim) and rounded to bf16.
  int32_t fold;
  int32_t rot_dim;
  float fold_scale;
  const float* fold_w;
};
// n = 1..3 independent copies (distinct destinations) in one launch.
hipError_t launch_row_copies(const RowCopyParams* jobs, int n, hipStream_t s);

hipError_t launch_kprep(const KPrepParams& p, hipStream_t s);
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, int32_t n_blocks,
                             hipStream_t s);
// True when launch_prefill takes the streaming kernel for short windows (which reads seg_steps and
// expects keys prepared with KPrepParams::fold set).
bool prefill_uses_swa(int window, int group, int rot_half);
// True when the streaming kernel can take key rows offset by qoff from the query rows (a cached
// context of qoff rows precedes the new ones): qoff = 0 or 63 (mod 64).
bool prefill_swa_offset_ok(int64_t qoff, int window);
hipError_t launch_prefill_swa(const PrefillParams& p, bool gated, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, int group, bool gated, hipStream_t s);
// The general tiled kernel only (any window, key rows offset from query rows, unfolded keys).
hipError_t launch_prefill_general(const PrefillParams& p, int group, bool gated, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);
// Size of the per-device static decode scratch, and its device address on the current device
// (looked up once per device; never the host-side symbol).
constexpr size_t kDecodeScratchBytes = size_t(96) << 20;
hipError_t decode_scratch_ptr(void** out);
hipError_t launch_rmsnorm(const RmsNormParams& p, hipStream_t s);
hipError_t launch_gemm(const GemmParams& p, hipStream_t s);
hipError_t launch_rmsnorm_fp8(const RmsNormFp8Params& p, hipStream_t s);
hipError_t launch_quant_rows(const QuantRowsParams& p, hipStream_t s);
hipError_t launch_gemm_fp8(const GemmFp8Params& p, hipStream_t s);

}  // namespace zg
