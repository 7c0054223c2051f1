// C ABI of the hybrid attention core: host-side validation, workspace planning and dispatch to the
// gfx950 kernels. Every argument is checked before anything is enqueued; failures return a
// zg_status and leave a thread-local message. No exception crosses the ABI.
#include "../../include/zg_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>

#include "zg_kernels.hpp"

namespace {

thread_local std::string g_err;

zg_status fail(zg_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
zg_status fail(zg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

zg_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ZG_OK;
  return fail(ZG_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int kD = 128;
constexpr int64_t kDecodeChunk = zg::kDecodeChunkKeys;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

zg_status check_cfg(const zg_attn_cfg* c) {
  if (!c) return fail(ZG_ERR_NULL, "cfg is NULL");
  if (c->n_q_heads < 1 || c->n_kv_heads < 1)
    return fail(ZG_ERR_SHAPE, "n_q_heads=%d n_kv_heads=%d must be >= 1", c->n_q_heads, c->n_kv_heads);
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(ZG_ERR_SHAPE, "n_q_heads=%d is not a multiple of n_kv_heads=%d", c->n_q_heads,
                c->n_kv_heads);
  const int g = c->n_q_heads / c->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(ZG_ERR_UNSUPPORTED, "query heads per KV head = %d; supported: 1, 2, 4, 8", g);
  if (c->head_dim != kD) return fail(ZG_ERR_UNSUPPORTED, "head_dim=%d; supported: 128", c->head_dim);
  if (c->window < 0) return fail(ZG_ERR_SHAPE, "window=%d must be >= 0", c->window);
  if (c->gated != 0 && c->gated != 1) return fail(ZG_ERR_SHAPE, "gated=%d must be 0 or 1", c->gated);
  if (c->rot_dim < 0 || c->rot_dim > 64 || (c->rot_dim & 1))
    return fail(ZG_ERR_UNSUPPORTED, "rot_dim=%d; supported: even values in [0, 64]", c->rot_dim);
  if (!(c->rope_base > 1.0) || !std::isfinite(c->rope_base))
    return fail(ZG_ERR_SHAPE, "rope_base=%g must be finite and > 1", c->rope_base);
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps))
    return fail(ZG_ERR_SHAPE, "rms_eps=%g must be finite and >= 0", (double)c->rms_eps);
  if (!std::isfinite(c->softmax_scale))
    return fail(ZG_ERR_SHAPE, "softmax_scale must be finite");
  return ZG_OK;
}

zg::RopeTableH rope_table(const zg_attn_cfg* c) {
  zg::RopeTableH t{};
  t.half = c->rot_dim / 2;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < t.half; ++i)
    t.rev[i] = std::pow(c->rope_base, -2.0 * i / (double)c->rot_dim) / two_pi;
  return t;
}

float scale_log2(const zg_attn_cfg* c) {
  const double s = c->softmax_scale > 0.f ? (double)c->softmax_scale : 1.0 / std::sqrt((double)kD);
  return (float)(s * 1.4426950408889634073599246810019);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// Runs of 64-query steps per workgroup of the banded streaming kernel, so that the grid roughly
// fills the device.
static int32_t swa_seg_steps(int64_t B, int64_t T, int64_t Hkv) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  const int64_t steps = (T + 63) / 64;
  const int64_t per_bh = B * Hkv;
  const int64_t n_seg = std::max<int64_t>(1, std::min<int64_t>(steps, cus / per_bh));
  return (int32_t)((steps + n_seg - 1) / n_seg);
}

extern "C" {

const char* zg_last_error(void) { return g_err.c_str(); }

uint64_t zg_kv_bytes(int32_t n_layers, int32_t global_every, int32_t n_kv_heads, int32_t head_dim,
                     int32_t window, int32_t elem_bytes, int64_t batch, int64_t seqlen) {
  if (n_layers < 0 || global_every < 0 || n_kv_heads < 0 || head_dim < 0 || window < 0 ||
      elem_bytes < 0 || batch < 0 || seqlen < 0) {
    fail(ZG_ERR_SHAPE, "zg_kv_bytes: arguments must be >= 0");
    return 0;
  }
  unsigned __int128 rows = 0;
  for (int32_t l = 1; l <= n_layers; ++l) {
    const bool global = window == 0 || (global_every > 0 && l % global_every == 0);
    rows += (unsigned __int128)(global ? seqlen : (seqlen < window ? seqlen : window));
  }
  const unsigned __int128 total = rows * 2u * (unsigned)n_kv_heads * (unsigned)head_dim *
                                  (unsigned)elem_bytes * (unsigned __int128)batch;
  if (total > std::numeric_limits<uint64_t>::max()) {
    fail(ZG_ERR_SHAPE, "zg_kv_bytes: result overflows uint64");
    return 0;
  }
  return (uint64_t)total;
}

size_t zg_attn_prefill_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T) {
  if (!cfg || B < 1 || T < 1 || cfg->n_kv_heads < 1) return 0;
  // k_hat, then the item counters of the tiled kernel's persistent launch
  return align256((size_t)B * T * cfg->n_kv_heads * kD * 2) + zg::kSchedBytes;
}

zg_status zg_attn_prefill(const zg_attn_cfg* cfg, int32_t B, int32_t T, int64_t pos0,
                          const void* q, const void* k, const void* v, const void* gate,
                          const float* q_norm_w, const float* k_norm_w,
                          const zg_token_strides* strides, void* out, void* workspace,
                          size_t workspace_bytes, void* stream) {
  try {
    zg_status st = check_cfg(cfg);
    if (st != ZG_OK) return st;
    if (!q || !k || !v || !out) return fail(ZG_ERR_NULL, "q, k, v and out must be non-NULL");
    if (cfg->gated && !gate) return fail(ZG_ERR_NULL, "gate must be non-NULL when gated=1");
    if (B < 1 || T < 1) return fail(ZG_ERR_SHAPE, "B=%d T=%d must be >= 1", B, T);
    if (pos0 < 0) return fail(ZG_ERR_SHAPE, "pos0=%lld must be >= 0", (long long)pos0);
    const int64_t Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads;
    if ((int64_t)B * T * Hq * kD >= (int64_t(1) << 40))
      return fail(ZG_ERR_SHAPE, "B*T*Hq*D too large");
    zg_token_strides s{Hq * kD, Hkv * kD, Hkv * kD, Hq * kD, Hq * kD};
    if (strides) s = *strides;
    if (s.q < Hq * kD || s.k < Hkv * kD || s.v < Hkv * kD || s.out < Hq * kD ||
        (cfg->gated && s.gate < Hq * kD) || (s.q | s.k | s.v | s.out) % 8 != 0 ||
        (cfg->gated && s.gate % 8 != 0))
      return fail(ZG_ERR_SHAPE, "token strides must be >= the packed row and multiples of 8");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (cfg->gated && !aligned16(gate)) || (q_norm_w && !aligned16(q_norm_w)) ||
        (k_norm_w && !aligned16(k_norm_w)))
      return fail(ZG_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    // q, K and V rows are fetched through 32-bit buffer offsets within one sequence's rows
    const int64_t max_row_bytes = 2 * std::max<int64_t>({s.q, s.v, Hkv * kD});
    if ((int64_t)(T + 64) * max_row_bytes >= (int64_t(1) << 32))
      return fail(ZG_ERR_UNSUPPORTED, "T * token stride of q or v (bytes) must stay below 4 GiB");
    const size_t need = zg_attn_prefill_workspace_bytes(cfg, B, T);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(ZG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                  workspace ? workspace_bytes : (size_t)0, need);
    if (!aligned16(workspace)) return fail(ZG_ERR_SHAPE, "workspace must be 16-byte aligned");

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const zg::RopeTableH rt = rope_table(cfg);
    zg::KPrepParams kp{};
    kp.k = static_cast<const uint16_t*>(k);
    kp.khat = static_cast<uint16_t*>(workspace);
    kp.k_norm_w = k_norm_w;
    kp.sk = s.k;
    kp.B = B;
    kp.T = T;
    kp.Hkv = (int32_t)Hkv;
    kp.pos0 = pos0;
    kp.out_rows = T;
    kp.out_row0 = 0;
    kp.eps = cfg->rms_eps;
    kp.rope = rt;
    const int G = (int)(Hq / Hkv);
    const int window = cfg->window >= T ? 0 : cfg->window;  // a window covering T is causal
    const bool swa = zg::prefill_uses_swa(window, G, rt.half);
    kp.fold = swa ? 1 : 0;
    kp.fold_scale = scale_log2(cfg);
    kp.fold_w = q_norm_w;
    // the item counters after k_hat, zeroed by this launch for the attention launch that follows
    uint32_t* counters = reinterpret_cast<uint32_t*>(
        static_cast<unsigned char*>(workspace) + align256((size_t)B * T * Hkv * kD * 2));
    kp.zero_words = counters;
    kp.n_zero_words = zg::kSchedWords;
    st = hip_status(zg::launch_kprep(kp, hs), "kprep launch");
    if (st != ZG_OK) return st;

    const int mq = 256 / G;
    zg::PrefillParams pp{};
    pp.q = static_cast<const uint16_t*>(q);
    pp.khat = static_cast<const uint16_t*>(workspace);
    pp.v = static_cast<const uint16_t*>(v);
    pp.gate = static_cast<const uint16_t*>(gate);
    pp.out = static_cast<uint16_t*>(out);
    pp.q_norm_w = q_norm_w;
    pp.sq = s.q;
    pp.sv = s.v;
    pp.sg = s.gate;
    pp.so = s.out;
    pp.B = B;
    pp.T = T;
    pp.Hq = (int32_t)Hq;
    pp.Hkv = (int32_t)Hkv;
    pp.pos0 = pos0;
    pp.window = window;
    pp.n_qtiles = (T + mq - 1) / mq;
    pp.kv_rows = T;
    pp.n_keys = T;
    pp.qoff = 0;
    pp.eps = cfg->rms_eps;
    pp.scale_log2 = scale_log2(cfg);
    pp.rope = rt;
    if ((int64_t)pp.n_qtiles * B * Hkv >= (int64_t(1) << 31))
      return fail(ZG_ERR_SHAPE, "grid too large");
    if (swa) pp.seg_steps = swa_seg_steps(B, T, Hkv);
    pp.counters = counters;
    return hip_status(zg::launch_prefill(pp, G, cfg->gated != 0, hs), "prefill launch");
  } catch (...) {
    return fail(ZG_ERR_HIP, "unexpected exception in zg_attn_prefill");
  }
}

// ---- training: forward with row log-sum-exp, and the backward pass ----
static zg_status check_train(const zg_attn_cfg* cfg, int32_t B, int32_t T) {
  zg_status st = check_cfg(cfg);
  if (st != ZG_OK) return st;
  if (cfg->n_q_heads != 4 * cfg->n_kv_heads)
    return fail(ZG_ERR_UNSUPPORTED, "training kernels: n_q_heads must be 4 * n_kv_heads (got %d / %d)",
                cfg->n_q_heads, cfg->n_kv_heads);
  if (B < 1 || T < 1) return fail(ZG_ERR_SHAPE, "B=%d T=%d must be >= 1", B, T);
  const int64_t Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads;
  if ((int64_t)B * T * Hq * kD >= (int64_t(1) << 40)) return fail(ZG_ERR_SHAPE, "B*T*Hq*D too large");
  // the forward kernel addresses one sequence's q, K and V rows through 32-bit byte offsets
  if ((int64_t)(T + 64) * 2 * Hq * kD >= (int64_t(1) << 32))
    return fail(ZG_ERR_UNSUPPORTED, "T * Hq * 256 bytes must stay below 4 GiB");
  if ((int64_t)((T + 63) / 64) * B * Hkv >= (int64_t(1) << 31)) return fail(ZG_ERR_SHAPE, "grid too large");
  return ZG_OK;
}

size_t zg_attn_forward_train_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T) {
  if (!cfg || B < 1 || T < 1 || cfg->n_kv_heads < 1) return 0;
  // k_hat for the tiled kernel, then the item counters of its persistent launch
  return align256((size_t)B * T * cfg->n_kv_heads * kD * 2) + zg::kSchedBytes;
}

zg_status zg_attn_forward_train(const zg_attn_cfg* cfg, int32_t B, int32_t T, const void* q,
                                const void* k, const void* v, const void* gate, void* out,
                                float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    zg_status st = check_train(cfg, B, T);
    if (st != ZG_OK) return st;
    if (!q || !k || !v || !out || !lse) return fail(ZG_ERR_NULL, "q, k, v, out and lse must be non-NULL");
    if (cfg->gated && !gate) return fail(ZG_ERR_NULL, "gate must be non-NULL when gated=1");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse) ||
        (cfg->gated && !aligned16(gate)))
      return fail(ZG_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    const size_t need = zg_attn_forward_train_workspace_bytes(cfg, B, T);
    if (!workspace || workspace_bytes < need)
      return fail(ZG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                  workspace ? workspace_bytes : (size_t)0, need);
    if (!aligned16(workspace)) return fail(ZG_ERR_SHAPE, "workspace must be 16-byte aligned");
    const int64_t Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const zg::RopeTableH rt = rope_table(cfg);
    zg::KPrepParams kp{};
    kp.k = static_cast<const uint16_t*>(k);
    kp.khat = static_cast<uint16_t*>(workspace);
    kp.sk = Hkv * kD;
    kp.B = B;
    kp.T = T;
    kp.Hkv = (int32_t)Hkv;
    kp.out_rows = T;
    kp.eps = cfg->rms_eps;
    kp.rope = rt;
    // the same kernel choice as a plain prefill: local layers of 4 heads per KV head run the banded
    // streaming kernel on folded keys, everything else the general tiled kernel
    const int window = cfg->window >= T ? 0 : cfg->window;  // a window covering T is causal
    const bool swa = zg::prefill_uses_swa(window, 4, rt.half);
    kp.fold = swa ? 1 : 0;
    kp.fold_scale = scale_log2(cfg);
    uint32_t* counters = reinterpret_cast<uint32_t*>(
        static_cast<unsigned char*>(workspace) + align256((size_t)B * T * Hkv * kD * 2));
    kp.zero_words = counters;
    kp.n_zero_words = zg::kSchedWords;
    st = hip_status(zg::launch_kprep(kp, hs), "kprep launch");
    if (st != ZG_OK) return st;
    zg::PrefillParams pp{};
    pp.q = static_cast<const uint16_t*>(q);
    pp.khat = static_cast<const uint16_t*>(workspace);
    pp.v = static_cast<const uint16_t*>(v);
    pp.gate = static_cast<const uint16_t*>(gate);
    pp.out = static_cast<uint16_t*>(out);
    pp.sq = Hq * kD;
    pp.sv = Hkv * kD;
    pp.sg = Hq * kD;
    pp.so = Hq * kD;
    pp.B = B;
    pp.T = T;
    pp.Hq = (int32_t)Hq;
    pp.Hkv = (int32_t)Hkv;
    pp.window = window;
    pp.n_qtiles = (T + 63) / 64;
    pp.kv_rows = T;
    pp.n_keys = T;
    pp.lse = lse;
    pp.eps = cfg->rms_eps;
    pp.scale_log2 = scale_log2(cfg);
    pp.rope = rt;
    if (swa) pp.seg_steps = swa_seg_steps(B, T, Hkv);
    pp.counters = counters;
    return hip_status(zg::launch_prefill(pp, 4, cfg->gated != 0, hs), "prefill launch");
  } catch (...) {
    return fail(ZG_ERR_HIP, "unexpected exception in zg_attn_forward_train");
  }
}

size_t zg_attn_backward_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T) {
  if (!cfg || B < 1 || T < 1 || cfg->n_q_heads < 1 || cfg->n_kv_heads < 1) return 0;
  const size_t bt = (size_t)B * T, hq = cfg->n_q_heads, hk = cfg->n_kv_heads;
  return 2 * align256(bt * hq * kD * 2) + align256(bt * hk * kD * 2) + align256(bt * hq * 16 * 2);
}

zg_status zg_attn_backward(const zg_attn_cfg* cfg, int32_t B, int32_t T, const void* q,
                           const void* k, const void* v, const void* gate, const void* out,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           void* dgate, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    zg_status st = check_train(cfg, B, T);
    if (st != ZG_OK) return st;
    if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
      return fail(ZG_ERR_NULL, "q, k, v, out, dout, lse, dq, dk and dv must be non-NULL");
    if (cfg->gated && (!gate || !dgate))
      return fail(ZG_ERR_NULL, "gate and dgate must be non-NULL when gated=1");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) ||
        !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        (cfg->gated && (!aligned16(gate) || !aligned16(dgate))))
      return fail(ZG_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    const size_t need = zg_attn_backward_workspace_bytes(cfg, B, T);
    if (!workspace || workspace_bytes < need)
      return fail(ZG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                  workspace ? workspace_bytes : (size_t)0, need);
    if (!aligned16(workspace)) return fail(ZG_ERR_SHAPE, "workspace must be 16-byte aligned");
    const int64_t Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads;
    const size_t bt = (size_t)B * T;
    char* ws = static_cast<char*>(workspace);
    zg::BwdParams bp{};
    bp.qc = reinterpret_cast<uint16_t*>(ws);
    ws += align256(bt * Hq * kD * 2);
    bp.dO = reinterpret_cast<uint16_t*>(ws);
    ws += align256(bt * Hq * kD * 2);
    bp.khat = reinterpret_cast<uint16_t*>(ws);
    ws += align256(bt * Hkv * kD * 2);
    bp.aux = reinterpret_cast<uint16_t*>(ws);

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const zg::RopeTableH rt = rope_table(cfg);
    // q_hat * scale * log2 e and k_hat in bf16: the operands the forward multiplied
    zg::KPrepParams kp{};
    kp.k = static_cast<const uint16_t*>(q);
    kp.khat = bp.qc;
    kp.sk = Hq * kD;
    kp.B = B;
    kp.T = T;
    kp.Hkv = (int32_t)Hq;
    kp.out_rows = T;
    kp.eps = cfg->rms_eps;
    kp.rope = rt;
    kp.fold = 1;
    kp.fold_scale = scale_log2(cfg);
    st = hip_status(zg::launch_kprep(kp, hs), "kprep launch (q)");
    if (st != ZG_OK) return st;
    kp.k = static_cast<const uint16_t*>(k);
    kp.khat = bp.khat;
    kp.sk = Hkv * kD;
    kp.Hkv = (int32_t)Hkv;
    kp.fold = 0;
    kp.fold_scale = 1.f;
    st = hip_status(zg::launch_kprep(kp, hs), "kprep launch (k)");
    if (st != ZG_OK) return st;
    // without a gate dO is dy itself
    if (!cfg->gated) bp.dO = const_cast<uint16_t*>(static_cast<const uint16_t*>(dout));

    bp.q = static_cast<const uint16_t*>(q);
    bp.k = static_cast<const uint16_t*>(k);
    bp.v = static_cast<const uint16_t*>(v);
    bp.gate = cfg->gated ? static_cast<const uint16_t*>(gate) : nullptr;
    bp.out = static_cast<const uint16_t*>(out);
    bp.dout = static_cast<const uint16_t*>(dout);
    bp.lse = lse;
    bp.dq = static_cast<uint16_t*>(dq);
    bp.dk = static_cast<uint16_t*>(dk);
    bp.dv = static_cast<uint16_t*>(dv);
    bp.dgate = cfg->gated ? static_cast<uint16_t*>(dgate) : nullptr;
    bp.B = B;
    bp.T = T;
    bp.Hq = (int32_t)Hq;
    bp.Hkv = (int32_t)Hkv;
    bp.window = cfg->window >= T ? 0 : cfg->window;
    bp.gated = cfg->gated;
    bp.n_qtiles = (T + 31) / 32;  // bwd_q: 32 queries per workgroup
    bp.pos0 = 0;
    bp.eps = cfg->rms_eps;
    bp.scale = (float)(cfg->softmax_scale > 0.f ? (double)cfg->softmax_scale : 1.0 / std::sqrt((double)kD));
    bp.rope = rt;
    return hip_status(zg::launch_backward(bp, hs), "backward launch");
  } catch (...) {
    return fail(ZG_ERR_HIP, "unexpected exception in zg_attn_backward");
  }
}

size_t zg_attn_prefill_cached_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T) {
  if (!cfg || B < 1 || T < 1 || cfg->n_kv_heads < 1) return 0;
  if (cfg->window <= 0) return 0;  // linear caches: keys are read from the cache itself
  const size_t rows = (size_t)cfg->window - 1 + T;  // ring context + the new tokens
  const size_t row_bytes = (size_t)cfg->n_kv_heads * kD * 2;
  // staged K and V (the new rows reach the ring straight from the K prologue)
  return 2 * align256((size_t)B * rows * row_bytes);
}

zg_status zg_attn_prefill_cached(const zg_attn_cfg* cfg, int32_t B, int32_t T, int64_t pos0,
                                 const void* q, const void* k, const void* v, const void* gate,
                                 const float* q_norm_w, const float* k_norm_w,
                                 const zg_token_strides* strides, void* k_cache, void* v_cache,
                                 int64_t cache_stride, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  try {
    zg_status st = check_cfg(cfg);
    if (st != ZG_OK) return st;
    if (!q || !k || !v || !out || !k_cache || !v_cache)
      return fail(ZG_ERR_NULL, "q, k, v, out and the caches must be non-NULL");
    if (cfg->gated && !gate) return fail(ZG_ERR_NULL, "gate must be non-NULL when gated=1");
    if (B < 1 || T < 1) return fail(ZG_ERR_SHAPE, "B=%d T=%d must be >= 1", B, T);
    if (pos0 < 0 || pos0 + T >= (int64_t(1) << 31))
      return fail(ZG_ERR_SHAPE, "pos0=%lld out of range", (long long)pos0);
    const int64_t Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads;
    const int64_t W = cfg->window;
    const bool ring = W > 0;
    if (!ring && cache_stride < pos0 + T)
      return fail(ZG_ERR_SHAPE, "linear cache: cache_stride=%lld < pos0 + T=%lld",
                  (long long)cache_stride, (long long)(pos0 + T));
    if ((int64_t)B * T * Hq * kD >= (int64_t(1) << 40))
      return fail(ZG_ERR_SHAPE, "B*T*Hq*D too large");
    zg_token_strides s{Hq * kD, Hkv * kD, Hkv * kD, Hq * kD, Hq * kD};
    if (strides) s = *strides;
    if (s.q < Hq * kD || s.k < Hkv * kD || s.v < Hkv * kD || s.out < Hq * kD ||
        (cfg->gated && s.gate < Hq * kD) || (s.q | s.k | s.v | s.out) % 8 != 0 ||
        (cfg->gated && s.gate % 8 != 0))
      return fail(ZG_ERR_SHAPE, "token strides must be >= the packed row and multiples of 8");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        !aligned16(k_cache) || !aligned16(v_cache) || (cfg->gated && !aligned16(gate)) ||
        (q_norm_w && !aligned16(q_norm_w)) || (k_norm_w && !aligned16(k_norm_w)))
      return fail(ZG_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
    const int64_t row = Hkv * kD;  // elements per cache row
    const int64_t n_ctx = ring ? std::min<int64_t>(pos0, W - 1) : pos0;
    const int64_t n_keys = n_ctx + T;
    if ((n_keys + 64) * 2 * std::max<int64_t>({s.q, row}) >= (int64_t(1) << 32))
      return fail(ZG_ERR_UNSUPPORTED, "(context + T) * row bytes must stay below 4 GiB");
    const size_t need = zg_attn_prefill_cached_workspace_bytes(cfg, B, T);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(ZG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                  workspace ? workspace_bytes : (size_t)0, need);
    if (need > 0 && !aligned16(workspace)) return fail(ZG_ERR_SHAPE, "workspace must be 16-byte aligned");

    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    uint16_t* kc = static_cast<uint16_t*>(k_cache);
    uint16_t* vc = static_cast<uint16_t*>(v_cache);
    // keys and values the attention reads: the linear cache itself, or a staging copy of the
    // ring's context followed by the new tokens
    uint16_t* ks = kc;
    uint16_t* vs = vc;
    int64_t kv_rows = cache_stride, row0 = pos0;
    const zg::RopeTableH rt = rope_table(cfg);
    const int G = (int)(Hq / Hkv);
    const int window = (ring && W < n_keys) ? (int)W : 0;  // a window covering every key is causal
    // Rings whose context offset suits it run on the banded streaming kernel, which takes keys
    // with the softmax scale and the q-norm weights folded in: the context rows are folded as they
    // are gathered, and the K prologue writes the new rows' k_hat folded to the staging rows and
    // unfolded to the ring.
    const bool swa = ring && zg::prefill_uses_swa(window, G, rt.half) &&
                     zg::prefill_swa_offset_ok(n_ctx, window);
    if (ring) {
      ks = static_cast<uint16_t*>(workspace);
      vs = ks + align256((size_t)B * (W - 1 + T) * row * 2) / 2;
      kv_rows = n_keys;
      row0 = n_ctx;
    }
    // copies ahead of the attention, issued as one launch: the ring's context K and V into the
    // staging rows 0 .. n_ctx-1, the new tokens' v after them (or into the linear cache)
    zg::RowCopyParams pre[3];
    int n_pre = 0;
    if (ring) {
      if (n_ctx > 0) {
        for (int which = 0; which < 2; ++which) {
          zg::RowCopyParams g{};
          g.src = which ? vc : kc;
          g.dst = which ? vs : ks;
          g.src_bstride = W; g.dst_bstride = kv_rows;
          g.src_row0 = pos0 - n_ctx; g.dst_row0 = 0;
          g.src_stride = row; g.dst_stride = row;
          g.src_ring = W; g.dst_ring = 0;
          g.row_elems = (int32_t)row; g.rows = (int32_t)n_ctx; g.B = B;
          if (swa && which == 0) {
            g.fold = 1;
            g.rot_dim = 2 * rt.half;
            g.fold_scale = scale_log2(cfg);
            g.fold_w = q_norm_w;
          }
          pre[n_pre++] = g;
        }
      }
    }
    zg::RowCopyParams vcp{};
    vcp.src = static_cast<const uint16_t*>(v);
    vcp.dst = vs;
    vcp.src_bstride = T; vcp.dst_bstride = kv_rows;
    vcp.src_row0 = 0; vcp.dst_row0 = row0;
    vcp.src_stride = s.v; vcp.dst_stride = row;
    vcp.row_elems = (int32_t)row; vcp.rows = T; vcp.B = B;
    pre[n_pre++] = vcp;
    st = hip_status(zg::launch_row_copies(pre, n_pre, hs), "ring gather / v copy launch");
    if (st != ZG_OK) return st;
    zg::KPrepParams kp{};
    kp.k = static_cast<const uint16_t*>(k);
    kp.khat = ks;
    kp.k_norm_w = k_norm_w;
    kp.sk = s.k;
    kp.B = B;
    kp.T = T;
    kp.Hkv = (int32_t)Hkv;
    kp.pos0 = pos0;
    kp.out_rows = kv_rows;
    kp.out_row0 = row0;
    kp.eps = cfg->rms_eps;
    kp.rope = rt;
    if (swa) {
      kp.fold = 1;
      kp.fold_scale = scale_log2(cfg);
      kp.fold_w = q_norm_w;
    }
    if (ring) {
      // the ring keeps the last W positions; the gather launch above has read its context rows
      const int64_t first = std::max<int64_t>(pos0, pos0 + T - W);
      kp.ring_k = kc;
      kp.ring_v = vc;
      kp.ring_v_src = static_cast<const uint16_t*>(v);
      kp.ring_sv = s.v;
      kp.ring_w = (int32_t)W;
      kp.ring_t0 = (int32_t)(first - pos0);
    }
    st = hip_status(zg::launch_kprep(kp, hs), "kprep launch");
    if (st != ZG_OK) return st;

    const int mq = 256 / G;
    zg::PrefillParams pp{};
    pp.q = static_cast<const uint16_t*>(q);
    pp.khat = ks;
    pp.v = vs;
    pp.gate = static_cast<const uint16_t*>(gate);
    pp.out = static_cast<uint16_t*>(out);
    pp.q_norm_w = q_norm_w;
    pp.sq = s.q;
    pp.sv = row;
    pp.sg = s.gate;
    pp.so = s.out;
    pp.B = B;
    pp.T = T;
    pp.Hq = (int32_t)Hq;
    pp.Hkv = (int32_t)Hkv;
    pp.pos0 = pos0;
    pp.window = window;
    pp.n_qtiles = (T + mq - 1) / mq;
    pp.kv_rows = kv_rows;
    pp.n_keys = (int32_t)n_keys;
    pp.qoff = (int32_t)n_ctx;
    pp.eps = cfg->rms_eps;
    pp.scale_log2 = scale_log2(cfg);
    pp.rope = rt;
    if ((int64_t)pp.n_qtiles * B * Hkv >= (int64_t(1) << 31))
      return fail(ZG_ERR_SHAPE, "grid too large");
    if (swa) {
      pp.seg_steps = swa_seg_steps(B, T, Hkv);
      st = hip_status(zg::launch_prefill_swa(pp, cfg->gated != 0, hs), "prefill launch");
    } else {
      st = hip_status(zg::launch_prefill_general(pp, G, cfg->gated != 0, hs), "prefill launch");
    }
    if (st != ZG_OK) return st;
    return ZG_OK;
  } catch (...) {
    return fail(ZG_ERR_HIP, "unexpected exception in zg_attn_prefill_cached");
  }
}

size_t zg_attn_decode_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int64_t max_seqlen) {
  if (!cfg || B < 1 || max_seqlen < 1 || cfg->n_q_heads < 1) return 0;
  const int64_t keys = cfg->window > 0 ? std::min<int64_t>(cfg->window, max_seqlen) : max_seqlen;
  const int64_t n_chunks = (keys + kDecodeChunk - 1) / kDecodeChunk;
  size_t bytes = align256((size_t)B * cfg->n_q_heads * kD * 4);
  if (n_chunks > 1) bytes += align256((size_t)B * cfg->n_q_heads * n_chunks * 132 * 4);
  return bytes;
}

// Every decode argument check except the workspace's.
static zg_status decode_check(const zg_attn_cfg* cfg, int32_t B, int64_t cache_stride,
                              int64_t max_seqlen, const void* q_new, const void* k_new,
                              const void* v_new, const void* gate, const float* q_norm_w,
                              const float* k_norm_w, const void* k_cache, const void* v_cache,
                              bool fp8, float k_scale, float v_scale, const int32_t* seqlens,
                              const void* out) {
  zg_status st = check_cfg(cfg);
  if (st != ZG_OK) return st;
  if (!q_new || !k_new || !v_new || !k_cache || !v_cache || !seqlens || !out)
    return fail(ZG_ERR_NULL, "q_new, k_new, v_new, caches, seqlens and out must be non-NULL");
  if (cfg->gated && !gate) return fail(ZG_ERR_NULL, "gate must be non-NULL when gated=1");
  if (B < 1) return fail(ZG_ERR_SHAPE, "B=%d must be >= 1", B);
  if (max_seqlen < 1 || max_seqlen >= (int64_t(1) << 31))
    return fail(ZG_ERR_SHAPE, "max_seqlen=%lld out of range", (long long)max_seqlen);
  const int64_t keys = cfg->window > 0 ? std::min<int64_t>(cfg->window, max_seqlen) : max_seqlen;
  if ((keys + kDecodeChunk - 1) / kDecodeChunk > zg::kDecodeMaxChunks)
    return fail(ZG_ERR_UNSUPPORTED, "max_seqlen=%lld: at most %lld keys per sequence",
                (long long)max_seqlen, (long long)(kDecodeChunk * zg::kDecodeMaxChunks));
  if (cfg->window == 0 && cache_stride < max_seqlen)
    return fail(ZG_ERR_SHAPE, "linear cache: cache_stride=%lld < max_seqlen=%lld",
                (long long)cache_stride, (long long)max_seqlen);
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(ZG_ERR_SHAPE, "k_scale and v_scale must be finite and > 0");
  if (!aligned16(q_new) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || (q_norm_w && !aligned16(q_norm_w)) ||
      (k_norm_w && !aligned16(k_norm_w)))
    return fail(ZG_ERR_SHAPE, "tensor pointers must be 16-byte aligned");
  return ZG_OK;
}

static zg_status decode_impl(const zg_attn_cfg* cfg, int32_t B, int64_t cache_stride,
                             int64_t max_seqlen, const void* q_new, const void* k_new,
                             const void* v_new, const void* gate, const float* q_norm_w,
                             const float* k_norm_w, void* k_cache, void* v_cache, bool fp8,
                             float k_scale, float v_scale, const int32_t* seqlens, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  try {
    zg_status st = decode_check(cfg, B, cache_stride, max_seqlen, q_new, k_new, v_new, gate,
                                q_norm_w, k_norm_w, k_cache, v_cache, fp8, k_scale, v_scale,
                                seqlens, out);
    if (st != ZG_OK) return st;
    const size_t need = zg_attn_decode_workspace_bytes(cfg, B, max_seqlen);
    if (!workspace || workspace_bytes < need)
      return fail(ZG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                  workspace ? workspace_bytes : (size_t)0, need);
    if (!aligned16(workspace)) return fail(ZG_ERR_SHAPE, "workspace must be 16-byte aligned");

    const int64_t Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads;
    const int64_t keys = cfg->window > 0 ? std::min<int64_t>(cfg->window, max_seqlen) : max_seqlen;
    zg::DecodeParams p{};
    p.q_new = static_cast<const uint16_t*>(q_new);
    p.k_new = static_cast<const uint16_t*>(k_new);
    p.v_new = static_cast<const uint16_t*>(v_new);
    p.gate = static_cast<const uint16_t*>(gate);
    p.q_norm_w = q_norm_w;
    p.k_norm_w = k_norm_w;
    p.k_cache = static_cast<uint16_t*>(k_cache);
    p.v_cache = static_cast<uint16_t*>(v_cache);
    p.seqlens = seqlens;
    p.out = static_cast<uint16_t*>(out);
    p.qhat = static_cast<float*>(workspace);
    p.partial = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         align256((size_t)B * Hq * kD * 4));
    p.B = B;
    p.Hq = (int32_t)Hq;
    p.Hkv = (int32_t)Hkv;
    p.window = cfg->window;
    p.rows = cfg->window > 0 ? cfg->window : cache_stride;
    p.chunk = (int32_t)kDecodeChunk;
    p.n_chunks = (int32_t)((keys + kDecodeChunk - 1) / kDecodeChunk);
    p.gated = cfg->gated;
    p.eps = cfg->rms_eps;
    p.scale_log2 = scale_log2(cfg) * (fp8 ? k_scale : 1.0f);
    p.rope = rope_table(cfg);
    p.fp8 = fp8 ? 1 : 0;
    p.k_inv = 1.0f / k_scale;
    p.v_inv = 1.0f / v_scale;
    p.v_scale = v_scale;
    return hip_status(zg::launch_decode(p, reinterpret_cast<hipStream_t>(stream)), "decode launch");
  } catch (...) {
    return fail(ZG_ERR_HIP, "unexpected exception in decode");
  }
}

zg_status zg_attn_decode(const zg_attn_cfg* cfg, int32_t B, int64_t cache_stride,
                         int64_t max_seqlen, const void* q_new, const void* k_new,
                         const void* v_new, const void* gate, const float* q_norm_w,
                         const float* k_norm_w, void* k_cache, void* v_cache,
                         const int32_t* seqlens, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return decode_impl(cfg, B, cache_stride, max_seqlen, q_new, k_new, v_new, gate, q_norm_w,
                     k_norm_w, k_cache, v_cache, false, 1.f, 1.f, seqlens, out, workspace,
                     workspace_bytes, stream);
}

zg_status zg_attn_decode_fp8(const zg_attn_cfg* cfg, int32_t B, int64_t cache_stride,
                             int64_t max_seqlen, const void* q_new, const void* k_new,
                             const void* v_new, const void* gate, const float* q_norm_w,
                             const float* k_norm_w, void* k_cache, void* v_cache, float k_scale,
                             float v_scale, const int32_t* seqlens, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return decode_impl(cfg, B, cache_stride, max_seqlen, q_new, k_new, v_new, gate, q_norm_w,
                     k_norm_w, k_cache, v_cache, true, k_scale, v_scale, seqlens, out, workspace,
                     workspace_bytes, stream);
}

zg_status zg_attn_decode_noalloc(const zg_attn_cfg* cfg, int32_t B, int64_t cache_stride,
                                 int64_t max_seqlen, const void* q_new, const void* k_new,
                                 const void* v_new, const void* gate, const float* q_norm_w,
                                 const float* k_norm_w, void* k_cache, void* v_cache,
                                 const int32_t* seqlens, void* out, void* stream) {
  try {
    // every argument and the scratch limit are checked before anything touches the device
    zg_status st = decode_check(cfg, B, cache_stride, max_seqlen, q_new, k_new, v_new, gate,
                                q_norm_w, k_norm_w, k_cache, v_cache, false, 1.f, 1.f, seqlens,
                                out);
    if (st != ZG_OK) return st;
    const size_t need = zg_attn_decode_workspace_bytes(cfg, B, max_seqlen);
    if (need > zg::kDecodeScratchBytes)
      return fail(ZG_ERR_UNSUPPORTED,
                  "zg_attn_decode_noalloc: %zu bytes of scratch needed, the static scratch holds %zu "
                  "(B * n_q_heads * (128 + chunks * 132) * 4 bytes, chunks = keys / 1024 rounded up)",
                  need, zg::kDecodeScratchBytes);
    void* scratch = nullptr;
    st = hip_status(zg::decode_scratch_ptr(&scratch), "decode scratch address");
    if (st != ZG_OK) return st;
    return decode_impl(cfg, B, cache_stride, max_seqlen, q_new, k_new, v_new, gate, q_norm_w,
                       k_norm_w, k_cache, v_cache, false, 1.f, 1.f, seqlens, out, scratch,
                       zg::kDecodeScratchBytes, stream);
  } catch (...) {
    return fail(ZG_ERR_HIP, "unexpected exception in zg_attn_decode_noalloc");
  }
}

zg_status zg_kv_to_fp8(const void* src_bf16, void* dst_e4m3, int64_t n, float scale, void* stream) {
  if (!src_bf16 || !dst_e4m3) return fail(ZG_ERR_NULL, "src and dst must be non-NULL");
  if (n < 0 || n % 16 != 0) return fail(ZG_ERR_SHAPE, "n=%lld must be a non-negative multiple of 16", (long long)n);
  if (!(std::isfinite(scale) && scale > 0.f)) return fail(ZG_ERR_SHAPE, "scale must be finite and > 0");
  if (!aligned16(src_bf16) || !aligned16(dst_e4m3)) return fail(ZG_ERR_SHAPE, "pointers must be 16-byte aligned");
  zg::ToFp8Params p{static_cast<const uint16_t*>(src_bf16), static_cast<uint8_t*>(dst_e4m3), n,
                    1.0f / scale};
  return hip_status(zg::launch_to_fp8(p, reinterpret_cast<hipStream_t>(stream)), "to-fp8 launch");
}

zg_status zg_hbm_read_probe(const void* src, int64_t bytes, uint32_t* sink, int32_t n_blocks,
                            void* stream) {
  if (!src || !sink) return fail(ZG_ERR_NULL, "src and sink must be non-NULL");
  if (bytes < 16 || bytes % 16 != 0) return fail(ZG_ERR_SHAPE, "bytes=%lld must be a positive multiple of 16", (long long)bytes);
  if (n_blocks < 1 || n_blocks > (1 << 20)) return fail(ZG_ERR_SHAPE, "n_blocks=%d out of range", n_blocks);
  if (!aligned16(src)) return fail(ZG_ERR_SHAPE, "src must be 16-byte aligned");
  return hip_status(zg::launch_read_probe(src, bytes, sink, n_blocks, reinterpret_cast<hipStream_t>(stream)),
                    "read probe launch");
}

zg_status zg_rmsnorm(int64_t rows, int32_t dim, const float* x, const float* w, float eps,
                     void* y_bf16, void* stream) {
  if (!x || !y_bf16) return fail(ZG_ERR_NULL, "x and y must be non-NULL");
  if (rows < 1 || rows >= (int64_t(1) << 31) || dim < 8 || dim > 8192 || dim % 8 != 0)
    return fail(ZG_ERR_SHAPE, "rows=%lld dim=%d: need rows >= 1, dim %% 8 == 0, 8 <= dim <= 8192",
                (long long)rows, dim);
  if (!(eps >= 0.f)) return fail(ZG_ERR_SHAPE, "eps must be >= 0");
  if (!aligned16(x) || !aligned16(y_bf16)) return fail(ZG_ERR_SHAPE, "pointers must be 16-byte aligned");
  zg::RmsNormParams p{x, w, static_cast<uint16_t*>(y_bf16), rows, dim, eps};
  return hip_status(zg::launch_rmsnorm(p, reinterpret_cast<hipStream_t>(stream)), "rmsnorm launch");
}

zg_status zg_gemm_bf16(int64_t M, int32_t N, int32_t K, const void* x_bf16, const void* w_bf16,
                       float* residual, void* y_bf16, int64_t ldy, void* stream) {
  if (!x_bf16 || !w_bf16) return fail(ZG_ERR_NULL, "x and w must be non-NULL");
  if (!residual && !y_bf16) return fail(ZG_ERR_NULL, "one of residual / y must be non-NULL");
  if (M < 1 || N < 8 || K < 64 || K % 64 != 0 || N % 8 != 0)
    return fail(ZG_ERR_SHAPE, "M=%lld N=%d K=%d: need M >= 1, N %% 8 == 0, K %% 64 == 0",
                (long long)M, N, K);
  if (y_bf16 && ldy < N) return fail(ZG_ERR_SHAPE, "ldy=%lld < N=%d", (long long)ldy, N);
  if (K > (1 << 20) || ((M + 255) / 256) * ((N + 255) / 256) >= (int64_t(1) << 31))
    return fail(ZG_ERR_SHAPE, "problem too large (K <= 2^20, fewer than 2^31 tiles of 256 x 256)");
  if (!aligned16(x_bf16) || !aligned16(w_bf16)) return fail(ZG_ERR_SHAPE, "x and w must be 16-byte aligned");
  zg::GemmParams p{static_cast<const uint16_t*>(x_bf16), static_cast<const uint16_t*>(w_bf16),
                   residual, static_cast<uint16_t*>(y_bf16), ldy, M, N, K};
  return hip_status(zg::launch_gemm(p, reinterpret_cast<hipStream_t>(stream)), "gemm launch");
}

size_t zg_attn_layer_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T) {
  if (!cfg || B < 1 || T < 1 || cfg->n_q_heads < 1 || cfg->n_kv_heads < 1) return 0;
  const size_t bt = (size_t)B * T;
  const size_t hidden = (size_t)cfg->n_q_heads * kD;
  const size_t nqkvg = (size_t)(cfg->n_q_heads + 2 * cfg->n_kv_heads + (cfg->gated ? cfg->n_q_heads : 0)) * kD;
  return align256(bt * hidden * 2) + align256(bt * nqkvg * 2) +
         zg_attn_prefill_workspace_bytes(cfg, B, T);
}

zg_status zg_attn_layer(const zg_attn_cfg* cfg, int32_t B, int32_t T, float* x,
                        const void* w_qkvg, const void* w_o, const float* q_norm_w,
                        const float* k_norm_w, void* workspace, size_t workspace_bytes,
                        void* stream) {
  zg_status st = check_cfg(cfg);
  if (st != ZG_OK) return st;
  if (!x || !w_qkvg || !w_o) return fail(ZG_ERR_NULL, "x, w_qkvg and w_o must be non-NULL");
  if (B < 1 || T < 1) return fail(ZG_ERR_SHAPE, "B=%d T=%d must be >= 1", B, T);
  const size_t need = zg_attn_layer_workspace_bytes(cfg, B, T);
  if (!workspace || workspace_bytes < need)
    return fail(ZG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                workspace ? workspace_bytes : (size_t)0, need);
  const int64_t Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads;
  const int64_t hidden = Hq * kD;
  const int64_t nqkvg = (Hq + 2 * Hkv + (cfg->gated ? Hq : 0)) * kD;
  const int64_t bt = (int64_t)B * T;
  char* ws = static_cast<char*>(workspace);
  void* h = ws;                                                  // bf16 [bt, hidden], reused for attn out
  void* qkvg = ws + align256(bt * hidden * 2);                   // bf16 [bt, nqkvg]
  void* kws = ws + align256(bt * hidden * 2) + align256(bt * nqkvg * 2);
  const size_t kws_bytes = zg_attn_prefill_workspace_bytes(cfg, B, T);

  st = zg_rmsnorm(bt, (int32_t)hidden, x, nullptr, cfg->rms_eps, h, stream);
  if (st != ZG_OK) return st;
  st = zg_gemm_bf16(bt, (int32_t)nqkvg, (int32_t)hidden, h, w_qkvg, nullptr, qkvg, nqkvg, stream);
  if (st != ZG_OK) return st;
  const uint16_t* base = static_cast<const uint16_t*>(qkvg);
  zg_token_strides s{nqkvg, nqkvg, nqkvg, nqkvg, hidden};
  st = zg_attn_prefill(cfg, B, T, 0, base, base + Hq * kD, base + (Hq + Hkv) * kD,
                       cfg->gated ? base + (Hq + 2 * Hkv) * kD : nullptr, q_norm_w, k_norm_w, &s, h,
                       kws, kws_bytes, stream);
  if (st != ZG_OK) return st;
  return zg_gemm_bf16(bt, (int32_t)hidden, (int32_t)hidden, h, w_o, x, nullptr, 0, stream);
}


// ---- E4M3 projections ----
static zg_status check_rows_fp8(int64_t rows, int32_t dim) {
  if (rows < 1 || rows >= (int64_t(1) << 31) || dim < 16 || dim > 8192 || dim % 16 != 0)
    return fail(ZG_ERR_SHAPE, "rows=%lld dim=%d: need rows >= 1, dim %% 16 == 0, 16 <= dim <= 8192",
                (long long)rows, dim);
  return ZG_OK;
}

zg_status zg_rmsnorm_fp8(int64_t rows, int32_t dim, const float* x, const float* w, float eps,
                         void* y_fp8, float* y_scale, void* stream) {
  if (!x || !y_fp8 || !y_scale) return fail(ZG_ERR_NULL, "x, y and y_scale must be non-NULL");
  zg_status st = check_rows_fp8(rows, dim);
  if (st != ZG_OK) return st;
  if (!(eps >= 0.f)) return fail(ZG_ERR_SHAPE, "eps must be >= 0");
  if (!aligned16(x) || !aligned16(y_fp8) || !aligned16(y_scale))
    return fail(ZG_ERR_SHAPE, "pointers must be 16-byte aligned");
  zg::RmsNormFp8Params p{x, w, static_cast<uint8_t*>(y_fp8), y_scale, rows, dim, eps};
  return hip_status(zg::launch_rmsnorm_fp8(p, reinterpret_cast<hipStream_t>(stream)), "rmsnorm_fp8 launch");
}

zg_status zg_quant_rows_fp8(int64_t rows, int32_t dim, const void* x_bf16, int64_t ldx,
                            void* y_fp8, float* y_scale, void* stream) {
  if (!x_bf16 || !y_fp8 || !y_scale) return fail(ZG_ERR_NULL, "x, y and y_scale must be non-NULL");
  zg_status st = check_rows_fp8(rows, dim);
  if (st != ZG_OK) return st;
  if (ldx < dim || ldx % 8 != 0) return fail(ZG_ERR_SHAPE, "ldx=%lld must be >= dim and a multiple of 8", (long long)ldx);
  if (!aligned16(x_bf16) || !aligned16(y_fp8) || !aligned16(y_scale))
    return fail(ZG_ERR_SHAPE, "pointers must be 16-byte aligned");
  zg::QuantRowsParams p{static_cast<const uint16_t*>(x_bf16), ldx, static_cast<uint8_t*>(y_fp8),
                        y_scale, rows, dim};
  return hip_status(zg::launch_quant_rows(p, reinterpret_cast<hipStream_t>(stream)), "quant_rows launch");
}

zg_status zg_gemm_fp8(int64_t M, int32_t N, int32_t K, const void* x_fp8, const float* x_scale,
                      const void* w_fp8, const float* w_scale, float* residual, void* y_bf16,
                      int64_t ldy, void* stream) {
  if (!x_fp8 || !x_scale || !w_fp8 || !w_scale)
    return fail(ZG_ERR_NULL, "x, x_scale, w and w_scale must be non-NULL");
  if (!residual && !y_bf16) return fail(ZG_ERR_NULL, "one of residual / y must be non-NULL");
  if (M < 1 || N < 8 || K < 128 || K % 128 != 0 || N % 8 != 0)
    return fail(ZG_ERR_SHAPE, "M=%lld N=%d K=%d: need M >= 1, N %% 8 == 0, K %% 128 == 0",
                (long long)M, N, K);
  if (y_bf16 && ldy < N) return fail(ZG_ERR_SHAPE, "ldy=%lld < N=%d", (long long)ldy, N);
  if (K > (1 << 20) || ((M + 255) / 256) * ((N + 255) / 256) >= (int64_t(1) << 31))
    return fail(ZG_ERR_SHAPE, "problem too large (K <= 2^20, fewer than 2^31 tiles of 256 x 256)");
  if (!aligned16(x_fp8) || !aligned16(w_fp8)) return fail(ZG_ERR_SHAPE, "x and w must be 16-byte aligned");
  zg::GemmFp8Params p{static_cast<const uint8_t*>(x_fp8), x_scale, static_cast<const uint8_t*>(w_fp8),
                      w_scale, residual, static_cast<uint16_t*>(y_bf16), ldy, M, N, K};
  return hip_status(zg::launch_gemm_fp8(p, reinterpret_cast<hipStream_t>(stream)), "gemm_fp8 launch");
}

size_t zg_attn_layer_fp8_workspace_bytes(const zg_attn_cfg* cfg, int32_t B, int32_t T) {
  if (!cfg || B < 1 || T < 1 || cfg->n_q_heads < 1 || cfg->n_kv_heads < 1) return 0;
  const size_t bt = (size_t)B * T;
  const size_t hidden = (size_t)cfg->n_q_heads * kD;
  const size_t nqkvg = (size_t)(cfg->n_q_heads + 2 * cfg->n_kv_heads + (cfg->gated ? cfg->n_q_heads : 0)) * kD;
  return align256(bt * hidden) + align256(bt * 4) + align256(bt * nqkvg * 2) +
         align256(bt * hidden * 2) + zg_attn_prefill_workspace_bytes(cfg, B, T);
}

zg_status zg_attn_layer_fp8(const zg_attn_cfg* cfg, int32_t B, int32_t T, float* x,
                            const void* w_qkvg_fp8, const float* s_qkvg, const void* w_o_fp8,
                            const float* s_o, const float* q_norm_w, const float* k_norm_w,
                            void* workspace, size_t workspace_bytes, void* stream) {
  zg_status st = check_cfg(cfg);
  if (st != ZG_OK) return st;
  if (!x || !w_qkvg_fp8 || !s_qkvg || !w_o_fp8 || !s_o)
    return fail(ZG_ERR_NULL, "x, w_qkvg, s_qkvg, w_o and s_o must be non-NULL");
  if (B < 1 || T < 1) return fail(ZG_ERR_SHAPE, "B=%d T=%d must be >= 1", B, T);
  const size_t need = zg_attn_layer_fp8_workspace_bytes(cfg, B, T);
  if (!workspace || workspace_bytes < need)
    return fail(ZG_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed",
                workspace ? workspace_bytes : (size_t)0, need);
  const int64_t Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads;
  const int64_t hidden = Hq * kD;
  const int64_t nqkvg = (Hq + 2 * Hkv + (cfg->gated ? Hq : 0)) * kD;
  const int64_t bt = (int64_t)B * T;
  char* ws = static_cast<char*>(workspace);
  void* hq = ws;                                         // E4M3 [bt, hidden]: h, then attn out
  float* sx = reinterpret_cast<float*>(ws + align256(bt * hidden));  // their row scales
  char* ws2 = ws + align256(bt * hidden) + align256(bt * 4);
  void* qkvg = ws2;                                      // bf16 [bt, nqkvg]
  void* attn = ws2 + align256(bt * nqkvg * 2);           // bf16 [bt, hidden]
  void* kws = ws2 + align256(bt * nqkvg * 2) + align256(bt * hidden * 2);
  const size_t kws_bytes = zg_attn_prefill_workspace_bytes(cfg, B, T);

  st = zg_rmsnorm_fp8(bt, (int32_t)hidden, x, nullptr, cfg->rms_eps, hq, sx, stream);
  if (st != ZG_OK) return st;
  st = zg_gemm_fp8(bt, (int32_t)nqkvg, (int32_t)hidden, hq, sx, w_qkvg_fp8, s_qkvg, nullptr, qkvg,
                   nqkvg, stream);
  if (st != ZG_OK) return st;
  const uint16_t* base = static_cast<const uint16_t*>(qkvg);
  zg_token_strides s{nqkvg, nqkvg, nqkvg, nqkvg, hidden};
  st = zg_attn_prefill(cfg, B, T, 0, base, base + Hq * kD, base + (Hq + Hkv) * kD,
                       cfg->gated ? base + (Hq + 2 * Hkv) * kD : nullptr, q_norm_w, k_norm_w, &s,
                       attn, kws, kws_bytes, stream);
  if (st != ZG_OK) return st;
  st = zg_quant_rows_fp8(bt, (int32_t)hidden, attn, hidden, hq, sx, stream);
  if (st != ZG_OK) return st;
  return zg_gemm_fp8(bt, (int32_t)hidden, (int32_t)hidden, hq, sx, w_o_fp8, s_o, x, nullptr, 0, stream);
}

}  // extern "C"
