// Decode for gfx950: one new token per sequence over a ring (local layers) or linear (global layers)
// KV cache of normalised, rotated keys. ZGCM-1 zh-TW translation page, section 2.3 "KV cache
// analysis": local layers keep a fixed 128-token window, global layers the whole sequence; decoding
// is memory-bandwidth bound.
//
// Three launches on the caller's stream:
//  1. decode_prep: RMSNorm + RoPE of q_new (kept as bf16-rounded fp32 in the workspace) and of k_new
//     (written into its cache row with v_new). Stream order makes the new row visible to step 2.
//  2. decode_attn: split-KV. One workgroup per (sequence, KV head, chunk of keys). Pass A streams the
//     chunk's K rows (16 lanes x 16 bytes per row) and forms the G scores of every key; the chunk's
//     softmax is then exact (max, exp2, sum over LDS); pass B streams the V rows and accumulates
//     P V. A sequence with one chunk writes its output directly; otherwise the chunk writes
//     (max, sum, unnormalised o) partials.
//  3. decode_combine: log-sum-exp merge of the partials, gate, bf16 store.
#include "zg_common.hpp"

namespace zg {

namespace {
constexpr int kDecThreads = 256;
constexpr int kPartStride = 132;  // floats per partial record: m, l, pad, pad, o[128]
constexpr int kMaxChunks = 1024;  // chunks per sequence the combine kernel merges

__device__ __forceinline__ int64_t n_valid_rows(int pos, int window) {
  return window > 0 ? (int64_t)min(pos + 1, window) : (int64_t)pos + 1;
}

// Sum over the 16 lanes of a DPP row, left in every lane: rotations by 8, 4, 2 and 1 (VALU only).
__device__ __forceinline__ float row16_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
  return v;
}
}  // namespace

__global__ __launch_bounds__(256) void decode_prep_kernel(DecodeParams p) {
  __shared__ float stage[128 * 64];
  const int b = blockIdx.x;
  const int pos = p.seqlens[b] - 1;
  // a length outside [1, cache rows] is a caller error: touch nothing (the output is unspecified)
  if (pos < 0 || (p.window == 0 && pos >= p.rows)) return;
  const int64_t row = p.window > 0 ? (int64_t)(pos % p.window) : (int64_t)pos;
  const int pair = threadIdx.x >> 1;
  const int half = threadIdx.x & 1;
  const int n_rows = p.Hq + p.Hkv;
  for (int r0 = 0; r0 < n_rows; r0 += 128) {
    const int r = r0 + pair;
    if (r < n_rows) {
      const bool is_q = r < p.Hq;
      const int h = is_q ? r : r - p.Hq;
      const uint16_t* src = is_q ? p.q_new + ((int64_t)b * p.Hq + h) * kHeadDim
                                 : p.k_new + ((int64_t)b * p.Hkv + h) * kHeadDim;
      float x[64];
      const u32x4* s4 = reinterpret_cast<const u32x4*>(src + 64 * half);
#pragma unroll
      for (int i = 0; i < 8; ++i) unpack8(s4[i], x + 8 * i);
      norm_rope_row(x, half, is_q ? p.q_norm_w : p.k_norm_w, p.eps, pos, p.rope, stage, pair,
                    128);
      if (is_q) {
        f32x4* dst = reinterpret_cast<f32x4*>(p.qhat + ((int64_t)b * p.Hq + h) * kHeadDim + 64 * half);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          // round to bf16 like the prefill matrix-core operand, keep as fp32
          const uint32_t w0 = pack_bf16(x[4 * i], x[4 * i + 1]);
          const uint32_t w1 = pack_bf16(x[4 * i + 2], x[4 * i + 3]);
          dst[i] = f32x4{bf16lo(w0), bf16hi(w0), bf16lo(w1), bf16hi(w1)};
        }
      } else {
        const int64_t off = ((int64_t)b * p.rows + row) * p.Hkv * kHeadDim + (int64_t)h * kHeadDim;
        u32x4* kd = reinterpret_cast<u32x4*>(p.k_cache + off + 64 * half);
#pragma unroll
        for (int i = 0; i < 8; ++i) kd[i] = pack8(x + 8 * i);
        const u32x4* vs = reinterpret_cast<const u32x4*>(
            p.v_new + ((int64_t)b * p.Hkv + h) * kHeadDim + 64 * half);
        u32x4* vd = reinterpret_cast<u32x4*>(p.v_cache + off + 64 * half);
#pragma unroll
        for (int i = 0; i < 8; ++i) vd[i] = vs[i];
      }
    }
    __syncthreads();
  }
}

template <int G>
__global__ __launch_bounds__(kDecThreads) void decode_attn_kernel(DecodeParams p) {
  constexpr int kMaxChunk = 1024;
  __shared__ float q_s[G][kHeadDim];
  __shared__ float s_s[G][kMaxChunk];
  __shared__ float red[4][G][kHeadDim];
  __shared__ float ml[G][2];

  const int chunk_id = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int pos = p.seqlens[b] - 1;
  if (pos < 0 || (p.window == 0 && pos >= p.rows)) return;
  const int64_t n_valid = min(n_valid_rows(pos, p.window), (int64_t)p.n_chunks * p.chunk);
  const int64_t k0 = (int64_t)chunk_id * p.chunk;
  if (k0 >= n_valid) return;
  const int n = (int)min((int64_t)p.chunk, n_valid - k0);
  const int n_chunks_b = (int)((n_valid + p.chunk - 1) / p.chunk);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = tid >> 4;   // key slot 0..15
  const int dl = tid & 15;   // 8-dim chunk

  for (int i = tid; i < G * kHeadDim; i += kDecThreads)
    q_s[i / kHeadDim][i % kHeadDim] =
        p.qhat[((int64_t)b * p.Hq + kvh * G) * kHeadDim + i];
  __syncthreads();
  float qv[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[h][j] = q_s[h][8 * dl + j];

  const int64_t row_stride = (int64_t)p.Hkv * kHeadDim;
  const uint16_t* kbase = p.k_cache + ((int64_t)b * p.rows + k0) * row_stride + kvh * kHeadDim + 8 * dl;
  const uint16_t* vbase = p.v_cache + ((int64_t)b * p.rows + k0) * row_stride + kvh * kHeadDim + 8 * dl;

  // ---- pass A: scores (log2 domain)
  constexpr int U = 4;
  for (int j0 = 0; j0 < n; j0 += 16 * U) {
    u32x4 kr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 16 * u + kg;
      kr[u] = j < n ? *reinterpret_cast<const u32x4*>(kbase + (int64_t)j * row_stride)
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kx[8];
      unpack8(kr[u], kx);
      float d[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a += qv[h][e] * kx[e];
        d[h] = a;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) d[h] = row16_sum(d[h]);
      const int j = j0 + 16 * u + kg;
      if (j < n && dl < G) {
        float v = d[0];
#pragma unroll
        for (int h = 1; h < G; ++h) v = (dl == h) ? d[h] : v;
        s_s[dl][j] = v * p.scale_log2;
      }
    }
  }
  __syncthreads();

  // ---- exact softmax over the chunk: one wave per head
  for (int h = wave; h < G; h += 4) {
    float mx = -INFINITY;
    for (int j = lane; j < n; j += 64) mx = fmaxf(mx, s_s[h][j]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
    float sum = 0.f;
    for (int j = lane; j < n; j += 64) {
      const float e = __builtin_amdgcn_exp2f(s_s[h][j] - mx);
      s_s[h][j] = e;
      sum += e;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += shfl_xor_f(sum, o);
    if (lane == 0) {
      ml[h][0] = mx;
      ml[h][1] = sum;
    }
  }
  __syncthreads();

  // ---- pass B: o[h][d] = sum_j p[h][j] v[j][d]
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  for (int j0 = 0; j0 < n; j0 += 16 * U) {
    u32x4 vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 16 * u + kg;
      vr[u] = j < n ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)j * row_stride)
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + 16 * u + kg;
      if (j < n) {
        float vx[8];
        unpack8(vr[u], vx);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pj = s_s[h][j];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] += pj * vx[e];
        }
      }
    }
  }
  // reduce the 4 key slots of a wave (lanes 16 apart), then the 4 waves through LDS
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = acc[h][e];
      a += shfl_xor_f(a, 16);
      a += shfl_xor_f(a, 32);
      acc[h][e] = a;
    }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][h][8 * lane + e] = acc[h][e];
  }
  __syncthreads();

  for (int i = tid; i < G * kHeadDim; i += kDecThreads) {
    const int h = i / kHeadDim;
    const int d = i - h * kHeadDim;
    const float o = red[0][h][d] + red[1][h][d] + red[2][h][d] + red[3][h][d];
    const int head = kvh * G + h;
    if (n_chunks_b == 1) {
      float y = o / ml[h][1];
      if (p.gated) {
        const float g = bf16lo(p.gate[((int64_t)b * p.Hq + head) * kHeadDim + d]);
        y *= __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
      }
      p.out[((int64_t)b * p.Hq + head) * kHeadDim + d] = (uint16_t)(pack_bf16(y, 0.f) & 0xffffu);
    } else {
      float* rec = p.partial + (((int64_t)b * p.Hq + head) * p.n_chunks + chunk_id) * kPartStride;
      if (d == 0) {
        rec[0] = ml[h][0];
        rec[1] = ml[h][1];
      }
      rec[4 + d] = o;
    }
  }
}

// One workgroup per (head, sequence), one thread per output dim. The chunk weights exp2(m_c - M)
// are formed once (chunks spread over the threads) and shared through LDS; the per-dim sums then
// issue their loads independently of each other.
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeParams p) {
  __shared__ float w_s[kMaxChunks];
  __shared__ float red[2];
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int pos = p.seqlens[b] - 1;
  if (pos < 0 || (p.window == 0 && pos >= p.rows)) return;
  const int64_t n_valid = n_valid_rows(pos, p.window);
  const int nc = (int)min((n_valid + p.chunk - 1) / p.chunk, (int64_t)p.n_chunks);
  if (nc <= 1) return;
  const float* rec = p.partial + ((int64_t)b * p.Hq + head) * p.n_chunks * kPartStride;
  float mx = -INFINITY;
  for (int c = d; c < nc; c += 128) mx = fmaxf(mx, rec[(int64_t)c * kPartStride]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
  if ((d & 63) == 0) red[d >> 6] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  float lw = 0.f;
  for (int c = d; c < nc; c += 128) {
    const float w = __builtin_amdgcn_exp2f(rec[(int64_t)c * kPartStride] - mx);
    w_s[c] = w;
    lw += rec[(int64_t)c * kPartStride + 1] * w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lw += shfl_xor_f(lw, o);
  __syncthreads();  // every thread has read red[] above before it is reused
  if ((d & 63) == 0) red[d >> 6] = lw;
  __syncthreads();
  const float l = red[0] + red[1];
  float o0 = 0.f, o1 = 0.f;
  int c = 0;
  for (; c + 1 < nc; c += 2) {
    o0 += rec[(int64_t)c * kPartStride + 4 + d] * w_s[c];
    o1 += rec[(int64_t)(c + 1) * kPartStride + 4 + d] * w_s[c + 1];
  }
  if (c < nc) o0 += rec[(int64_t)c * kPartStride + 4 + d] * w_s[c];
  float y = (o0 + o1) / l;
  if (p.gated) {
    const float g = bf16lo(p.gate[((int64_t)b * p.Hq + head) * kHeadDim + d]);
    y *= __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
  }
  p.out[((int64_t)b * p.Hq + head) * kHeadDim + d] = (uint16_t)(pack_bf16(y, 0.f) & 0xffffu);
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(decode_prep_kernel, dim3(p.B), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = p.Hq / p.Hkv;
  const dim3 grid(p.n_chunks, p.Hkv, p.B);
  switch (G) {
    case 1: hipLaunchKernelGGL(decode_attn_kernel<1>, grid, dim3(kDecThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL(decode_attn_kernel<2>, grid, dim3(kDecThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL(decode_attn_kernel<4>, grid, dim3(kDecThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL(decode_attn_kernel<8>, grid, dim3(kDecThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.n_chunks > 1) {
    hipLaunchKernelGGL(decode_combine_kernel, dim3(p.Hq, p.B), dim3(128), 0, s, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace zg
