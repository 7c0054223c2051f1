// Decode for gfx950: one new token per sequence over a ring (local layers) or linear (global layers)
// KV cache of normalised, rotated keys. ZGCM-1 zh-TW translation page, section 2.3 "KV cache
// analysis": local layers keep a fixed 128-token window, global layers the whole sequence; decoding
// is memory-bandwidth bound.
//
// Three launches on the caller's stream:
//  1. decode_prep: RMSNorm + RoPE of q_new (kept as bf16-rounded fp32 in the workspace) and of k_new
//     (written into its cache row with v_new). Stream order makes the new row visible to step 2.
//  2. decode_attn: split-KV. One workgroup per (sequence, KV head, chunk of 1024 keys). Pass A
//     streams the chunk's K rows (8 lanes x 2 x 16 bytes per 256-byte row, non-temporal loads) and
//     forms the G scores of every key with v_dot2_f32_bf16 on bf16 pairs; the chunk's softmax is
//     then exact (max, exp2, sum over LDS) and leaves bf16 P in key pairs; pass B streams the V rows
//     (16 lanes x 16 bytes per row) and accumulates P V, again with v_dot2_f32_bf16 over key pairs.
//     A sequence with one chunk writes its output directly; otherwise the chunk writes (max, sum,
//     unnormalised o) partials.
//  3. decode_combine: log-sum-exp merge of the partials, gate, bf16 store.
#include <mutex>

#include "zg_mfma.hpp"

namespace zg {

namespace {
constexpr int kDecThreads = 256;
constexpr int kPartStride = 132;  // floats per partial record: m, l, pad, pad, o[128]

__device__ __forceinline__ int64_t n_valid_rows(int pos, int window) {
  return window > 0 ? (int64_t)min(pos + 1, window) : (int64_t)pos + 1;
}

// Sixteen floats times `inv` as E4M3 codes (pack4_e4m3), packed in element order.
__device__ __forceinline__ u32x4 pack16_e4m3(const float* x, float inv) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = pack4_e4m3(x[4 * i] * inv, x[4 * i + 1] * inv, x[4 * i + 2] * inv, x[4 * i + 3] * inv);
  return w;
}
// Two E4M3 bytes (word `hi` of w) widened exactly to a bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
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

// Prep of one decode step. For each sequence b (new token at pos = seqlens[b] - 1): the Hq query
// rows become q_hat (fp32 holding bf16-rounded values, workspace), the Hkv key rows become k_hat,
// written with v_new into cache row pos (ring slot pos % window). Sixteen lanes per 256-byte head
// row, lane c holding dims 8c..8c+7; a 256-thread block takes 16 rows of the flattened
// [B, Hq + Hkv] row list. The RMS sum is reduced over the row's lanes; RoPE pairs (i, i + h) are
// exchanged through the wave's LDS rows, lane c rotating pairs c and c + 16.
constexpr int kDpStage = 68;  // floats per staged row (64 used; padded)

__global__ __launch_bounds__(256) void decode_prep_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float stage[4][4][kDpStage];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4;
  const int c = lane & 15;
  const int n_rows = p.Hq + p.Hkv;
  const int64_t rg = (int64_t)blockIdx.x * 16 + wave * 4 + grp;  // flattened (b, row)
  const bool in_range = rg < (int64_t)p.B * n_rows;
  const int b = in_range ? (int)(rg / n_rows) : 0;
  const int r = (int)(rg - (int64_t)b * n_rows);
  const int pos = in_range ? p.seqlens[b] - 1 : -1;
  // a length outside [1, cache rows] is a caller error: touch nothing (the output is unspecified)
  const bool valid = in_range && pos >= 0 && (p.window > 0 || pos < p.rows);
  const bool is_q = r < p.Hq;
  const int h = is_q ? r : r - p.Hq;
  const int hr = p.rope.half;
  const int rot = 2 * hr;

  const uint16_t* src = is_q ? p.q_new + ((int64_t)b * p.Hq + h) * kHeadDim
                             : p.k_new + ((int64_t)b * p.Hkv + h) * kHeadDim;
  float x[8];
  unpack8(valid ? *reinterpret_cast<const u32x4*>(src + 8 * c) : u32x4{0u, 0u, 0u, 0u}, x);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
  ss = row16_sum(ss);
  const float inv = rsqrtf(ss * (1.0f / kHeadDim) + p.eps);
  const float* w = is_q ? p.q_norm_w : p.k_norm_w;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] *= inv * (w ? w[8 * c + j] : 1.0f);
  if (hr > 0) {
    double rev0 = 0.0, rev1 = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (c == j) {
        rev0 = p.rope.rev[j];
        rev1 = p.rope.rev[j + 16];
      }
    }
    float* sr = &stage[wave][grp][0];
    const bool rotates = 8 * c < rot;
    if (rotates) {
      *reinterpret_cast<f32x4*>(sr + 8 * c) = f32x4{x[0], x[1], x[2], x[3]};
      *reinterpret_cast<f32x4*>(sr + 8 * c + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS ops complete in order
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pi = c + 16 * k;
      if (pi < hr) {
        float cs, sn;
        rope_cs(pos, k ? rev1 : rev0, cs, sn);
        const float a = sr[pi];
        const float bb = sr[pi + hr];
        sr[pi] = a * cs - bb * sn;
        sr[pi + hr] = bb * cs + a * sn;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (rotates) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(sr + 8 * c);
      const f32x4 hi4 = *reinterpret_cast<const f32x4*>(sr + 8 * c + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = lo[j];
        x[4 + j] = hi4[j];
      }
    }
  }
  if (!valid) return;
  if (is_q) {
    // round to bf16 like the prefill matrix-core operand, keep as fp32
    f32x4* dst = reinterpret_cast<f32x4*>(p.qhat + ((int64_t)b * p.Hq + h) * kHeadDim + 8 * c);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t w0 = pack_bf16(x[4 * i], x[4 * i + 1]);
      const uint32_t w1 = pack_bf16(x[4 * i + 2], x[4 * i + 3]);
      dst[i] = f32x4{bf16lo(w0), bf16hi(w0), bf16lo(w1), bf16hi(w1)};
    }
    return;
  }
  const int64_t row = p.window > 0 ? (int64_t)(pos % p.window) : (int64_t)pos;
  const int64_t off = ((int64_t)b * p.rows + row) * p.Hkv * kHeadDim + (int64_t)h * kHeadDim + 8 * c;
  const u32x4 vw = *reinterpret_cast<const u32x4*>(p.v_new + ((int64_t)b * p.Hkv + h) * kHeadDim + 8 * c);
  if (!p.fp8) {
    *reinterpret_cast<u32x4*>(p.k_cache + off) = pack8(x);
    *reinterpret_cast<u32x4*>(p.v_cache + off) = vw;
  } else {
    // E4M3 rows: one byte per element
    float vf[8];
    unpack8(vw, vf);
    const float ki = p.k_inv, vi = p.v_inv;
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(p.k_cache) + off) =
        u32x2{pack4_e4m3(x[0] * ki, x[1] * ki, x[2] * ki, x[3] * ki),
              pack4_e4m3(x[4] * ki, x[5] * ki, x[6] * ki, x[7] * ki)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(p.v_cache) + off) =
        u32x2{pack4_e4m3(vf[0] * vi, vf[1] * vi, vf[2] * vi, vf[3] * vi),
              pack4_e4m3(vf[4] * vi, vf[5] * vi, vf[6] * vi, vf[7] * vi)};
  }
}

constexpr int kDecKL = 8;  // lanes per key row in pass A
constexpr int kDecLA = 8;  // 16-byte K loads in flight per lane in pass A

namespace {
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         c, false);
}

// Sum over groups of KL consecutive lanes (KL = 4, 8 or 16), left in every lane of the group.
template <int KL>
__device__ __forceinline__ float group_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  if constexpr (KL >= 8)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
  if constexpr (KL >= 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false));
  return v;
}

// Cache rows are read once per step: non-temporal loads keep them from displacing reused lines.
__device__ __forceinline__ u32x4 stream_load(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

}  // namespace

template <int G>
__global__ __launch_bounds__(kDecThreads) void decode_attn_kernel(DecodeParams p) {
  constexpr int kMaxChunk = kDecodeChunkKeys;
  constexpr int KL = kDecKL;
  constexpr int CPK = 16 / KL;          // 16-byte pieces of a 256-byte key row per lane (pass A)
  constexpr int KPR = kDecThreads / KL;  // keys per workgroup round (pass A)
  constexpr int UA = kDecLA / CPK > 0 ? kDecLA / CPK : 1;  // rounds per pass-A step
  constexpr int STEP_A = KPR * UA;       // keys per pass-A step
  static_assert(KL == 4 || KL == 8 || KL == 16, "lanes per key");
  static_assert(kMaxChunk % 64 == 0, "pass B walks the chunk in blocks of 64 keys");
  static_assert(G * kMaxChunk >= 4 * G * kHeadDim, "the score rows also hold the final reduction");
  // Head h's row of s_s holds its raw scores; the softmax then overwrites the row's first half
  // with bf16 P in key pairs (dword q <- keys of pair q, read before any later write reaches
  // them); after pass B the array holds the cross-wave reduction.
  __shared__ float s_s[G * kMaxChunk];
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
  const int64_t row_stride = (int64_t)p.Hkv * kHeadDim;
  const int64_t head_off = ((int64_t)b * p.rows + k0) * row_stride + kvh * kHeadDim;

  // ---- pass A: raw scores q.k (bf16 pairs through v_dot2_f32_bf16, fp32 sums)
  {
    const int kq = tid / KL;
    const int sub = tid % KL;
    uint32_t qp[G][CPK][4];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < CPK; ++c) {
        const f32x4* src = reinterpret_cast<const f32x4*>(
            p.qhat + ((int64_t)b * p.Hq + kvh * G + h) * kHeadDim + 8 * sub + 8 * KL * c);
        const f32x4 a = src[0], bb = src[1];
        qp[h][c][0] = pack_bf16(a[0], a[1]);
        qp[h][c][1] = pack_bf16(a[2], a[3]);
        qp[h][c][2] = pack_bf16(bb[0], bb[1]);
        qp[h][c][3] = pack_bf16(bb[2], bb[3]);
      }
    const uint16_t* kbase = p.k_cache + head_off + 8 * sub;
    auto load = [&](u32x4 (&kr)[UA][CPK], int j0) {
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int j = j0 + KPR * u + kq;
#pragma unroll
        for (int c = 0; c < CPK; ++c)
          kr[u][c] = j < n ? stream_load(kbase + (int64_t)j * row_stride + 8 * KL * c)
                           : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto score = [&](const u32x4 (&kr)[UA][CPK], int j0) {
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        float d[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.f;
#pragma unroll
          for (int c = 0; c < CPK; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t w = kr[u][c][i];
              a = dot2(w, qp[h][c][i], a);
            }
          d[h] = group_sum<KL>(a);
        }
        const int j = j0 + KPR * u + kq;
#pragma unroll
        for (int h0 = 0; h0 < G; h0 += KL) {  // lane sub writes heads h0 + sub
          if (j < n && h0 + sub < G) {
            float v = d[h0];
#pragma unroll
            for (int h = h0 + 1; h < G && h < h0 + KL; ++h) v = (sub == h - h0) ? d[h] : v;
            s_s[(h0 + sub) * kMaxChunk + j] = v;
          }
        }
      }
    };
    for (int j0 = 0; j0 < n; j0 += STEP_A) {
      u32x4 ka[UA][CPK];
      load(ka, j0);
      score(ka, j0);
    }
  }
  __syncthreads();

  // ---- exact softmax over the chunk, one wave per head; P rounded to bf16 and stored in key
  // pairs over the head's score row, the row sum taken over the rounded values. Pass B pairs key
  // j with key j + 16 (j % 32 < 16): dword (j / 64) * 32 + ((j / 32) % 2) * 16 + j % 16 holds both.
  const int n_pad = (n + 63) & ~63;
  for (int h = wave; h < G; h += 4) {
    float* sh = s_s + h * kMaxChunk;
    float mx = -INFINITY;
    for (int j = lane; j < n; j += 64) mx = fmaxf(mx, sh[j]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
    const float c = p.scale_log2;
    const float nmc = -mx * c;
    float sum = 0.f;
    for (int q = lane; q < n_pad / 2; q += 64) {
      const int ja = (q >> 5) * 64 + ((q >> 4) & 1) * 32 + (q & 15);  // ja >= q
      const int jb = ja + 16;
      const float ea = ja < n ? __builtin_amdgcn_exp2f(__builtin_fmaf(sh[ja], c, nmc)) : 0.f;
      const float eb = jb < n ? __builtin_amdgcn_exp2f(__builtin_fmaf(sh[jb], c, nmc)) : 0.f;
      const uint32_t w = pack_bf16(ea, eb);
      sh[q] = __uint_as_float(w);  // same element type as the score reads: no reordering across
      sum += bf16lo(w) + bf16hi(w);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += shfl_xor_f(sum, o);
    if (lane == 0) {
      ml[h][0] = mx * c;
      ml[h][1] = sum;
    }
  }
  __syncthreads();

  // ---- pass B: o[h][d] = sum_j p[h][j] v[j][d]; keys j and j + 16 of a lane paired per dim
  const int kg = tid >> 4;  // key slot 0..15
  const int dl = tid & 15;  // 8-dim piece of the row
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  const uint16_t* vbase = p.v_cache + head_off + 8 * dl;
  auto load_v = [&](u32x4 (&vr)[4], int j0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + 16 * u + kg;
      vr[u] = j < n ? stream_load(vbase + (int64_t)j * row_stride) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto accumulate = [&](const u32x4 (&vr)[4], int j0) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = vr[2 * t][i], bb = vr[2 * t + 1][i];
        lo[i] = __builtin_amdgcn_perm(bb, a, 0x05040100u);  // dim 2i of keys (j, j + 16)
        hi[i] = __builtin_amdgcn_perm(bb, a, 0x07060302u);  // dim 2i + 1
      }
      const int q = (j0 >> 6) * 32 + t * 16 + kg;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint32_t pw = __float_as_uint(s_s[h * kMaxChunk + q]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[h][2 * i] = dot2(lo[i], pw, acc[h][2 * i]);
          acc[h][2 * i + 1] = dot2(hi[i], pw, acc[h][2 * i + 1]);
        }
      }
    }
  };
  for (int j0 = 0; j0 < n; j0 += 64) {
    u32x4 va[4];
    load_v(va, j0);
    accumulate(va, j0);
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
  __syncthreads();  // every wave is done reading P
  float* red = s_s;  // [4 waves][G][128]
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[(wave * G + h) * kHeadDim + 8 * lane + e] = acc[h][e];
  }
  __syncthreads();

  for (int i = tid; i < G * kHeadDim; i += kDecThreads) {
    const int h = i / kHeadDim;
    const int d = i - h * kHeadDim;
    const float o = red[(0 * G + h) * kHeadDim + d] + red[(1 * G + h) * kHeadDim + d] +
                    red[(2 * G + h) * kHeadDim + d] + red[(3 * G + h) * kHeadDim + d];
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

// The same split-KV attention over E4M3 caches (128 bytes per key and head). Pass A: 8 lanes per
// key row, 16 bytes = 16 elements each; two elements at a time are widened exactly to a bf16 pair
// and enter v_dot2_f32_bf16 with the matching q pair. Pass B: 8 lanes per value row (16 elements);
// the E4M3 bytes of keys j and j + 32 are interleaved by v_perm_b32 before widening, so each bf16
// pair holds one element of both keys and meets that key pair's P. Stored values stand for value *
// scale: the key scale is folded into the score scale, the value scale applied to o.
template <int G>
__global__ __launch_bounds__(kDecThreads) void decode_attn_fp8_kernel(DecodeParams p) {
  constexpr int kMaxChunk = kDecodeChunkKeys;
  constexpr int KL = 8;                  // lanes per key row (pass A) and per value row (pass B)
  constexpr int KPR = kDecThreads / KL;  // 32 keys per workgroup round
  constexpr int UA = 8;                  // rounds per pass-A step
  static_assert(kMaxChunk % 128 == 0, "pass B walks the chunk in blocks of 128 keys");
  __shared__ float s_s[G * kMaxChunk];   // scores, then P pairs, then the cross-wave reduction
  __shared__ float ml[G][2];
  static_assert(G * kMaxChunk >= 4 * G * kHeadDim, "reduction fits the score rows");

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
  const int64_t row_stride = (int64_t)p.Hkv * kHeadDim;  // bytes
  const int64_t head_off = ((int64_t)b * p.rows + k0) * row_stride + kvh * kHeadDim;
  const uint8_t* kc = reinterpret_cast<const uint8_t*>(p.k_cache);
  const uint8_t* vc = reinterpret_cast<const uint8_t*>(p.v_cache);
  const int kq = tid / KL;
  const int sub = tid % KL;

  // ---- pass A: raw scores against the stored keys
  {
    uint32_t qp[G][8];  // q pairs of dims 16 sub + 2 i, + 1
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const f32x4* src = reinterpret_cast<const f32x4*>(
          p.qhat + ((int64_t)b * p.Hq + kvh * G + h) * kHeadDim + 16 * sub);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 a = src[i];
        qp[h][2 * i] = pack_bf16(a[0], a[1]);
        qp[h][2 * i + 1] = pack_bf16(a[2], a[3]);
      }
    }
    const uint8_t* kbase = kc + head_off + 16 * sub;
    for (int j0 = 0; j0 < n; j0 += KPR * UA) {
      u32x4 kr[UA];
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int j = j0 + KPR * u + kq;
        kr[u] = j < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + (int64_t)j * row_stride))
                      : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        uint32_t kp[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w = kr[u][i];
          kp[2 * i] = e4m3x2_bf16<false>(w);
          kp[2 * i + 1] = e4m3x2_bf16<true>(w);
        }
        float d[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) a = dot2(kp[i], qp[h][i], a);
          d[h] = group_sum<KL>(a);
        }
        const int j = j0 + KPR * u + kq;
#pragma unroll
        for (int h0 = 0; h0 < G; h0 += KL) {
          if (j < n && h0 + sub < G) {
            float v = d[h0];
#pragma unroll
            for (int h = h0 + 1; h < G && h < h0 + KL; ++h) v = (sub == h - h0) ? d[h] : v;
            s_s[(h0 + sub) * kMaxChunk + j] = v;
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- exact softmax over the chunk, one wave per head; bf16 P stored in key pairs (j, j + 32)
  // (j % 64 < 32) over the head's score row: dword (j / 64) * 32 + j % 32 holds both
  const int n_pad = (n + 127) & ~127;
  for (int h = wave; h < G; h += 4) {
    float* sh = s_s + h * kMaxChunk;
    float mx = -INFINITY;
    for (int j = lane; j < n; j += 64) mx = fmaxf(mx, sh[j]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
    const float c = p.scale_log2;
    const float nmc = -mx * c;
    float sum = 0.f;
    for (int q = lane; q < n_pad / 2; q += 64) {
      const int ja = (q >> 5) * 64 + (q & 31);  // ja >= q
      const int jb = ja + 32;
      const float ea = ja < n ? __builtin_amdgcn_exp2f(__builtin_fmaf(sh[ja], c, nmc)) : 0.f;
      const float eb = jb < n ? __builtin_amdgcn_exp2f(__builtin_fmaf(sh[jb], c, nmc)) : 0.f;
      const uint32_t w = pack_bf16(ea, eb);
      sh[q] = __uint_as_float(w);
      sum += bf16lo(w) + bf16hi(w);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += shfl_xor_f(sum, o);
    if (lane == 0) {
      ml[h][0] = mx * c;
      ml[h][1] = sum;
    }
  }
  __syncthreads();

  // ---- pass B: o[h][d] = sum_j p[h][j] v[j][d] over key pairs (j, j + 32)
  float acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
  const uint8_t* vbase = vc + head_off + 16 * sub;
  for (int j0 = 0; j0 < n; j0 += 128) {
    u32x4 vr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + 32 * u + kq;
      vr[u] = j < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + (int64_t)j * row_stride))
                    : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = (j0 >> 6) * 32 + 32 * t + kq;  // key pair (j0 + 64 t + kq, + 32)
      uint32_t pw[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pw[h] = __float_as_uint(s_s[h * kMaxChunk + q]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = vr[2 * t][i], bb = vr[2 * t + 1][i];  // dims 4 i .. 4 i + 3
        const uint32_t lo = __builtin_amdgcn_perm(bb, a, 0x05010400u);  // a0 b0 a1 b1
        const uint32_t hi = __builtin_amdgcn_perm(bb, a, 0x07030602u);  // a2 b2 a3 b3
        const uint32_t d0 = e4m3x2_bf16<false>(lo), d1 = e4m3x2_bf16<true>(lo);
        const uint32_t d2 = e4m3x2_bf16<false>(hi), d3 = e4m3x2_bf16<true>(hi);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          acc[h][4 * i] = dot2(d0, pw[h], acc[h][4 * i]);
          acc[h][4 * i + 1] = dot2(d1, pw[h], acc[h][4 * i + 1]);
          acc[h][4 * i + 2] = dot2(d2, pw[h], acc[h][4 * i + 2]);
          acc[h][4 * i + 3] = dot2(d3, pw[h], acc[h][4 * i + 3]);
        }
      }
    }
  }
  // reduce the 8 key slots of a wave (lanes 8 apart), then the 4 waves through LDS
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float a = acc[h][e];
      a += shfl_xor_f(a, 8);
      a += shfl_xor_f(a, 16);
      a += shfl_xor_f(a, 32);
      acc[h][e] = a;
    }
  __syncthreads();  // every wave is done reading P
  float* red = s_s;  // [4 waves][G][128]
  if (lane < 8) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[(wave * G + h) * kHeadDim + 16 * lane + e] = acc[h][e];
  }
  __syncthreads();

  for (int i = tid; i < G * kHeadDim; i += kDecThreads) {
    const int h = i / kHeadDim;
    const int d = i - h * kHeadDim;
    const float o = p.v_scale * (red[(0 * G + h) * kHeadDim + d] + red[(1 * G + h) * kHeadDim + d] +
                                 red[(2 * G + h) * kHeadDim + d] + red[(3 * G + h) * kHeadDim + d]);
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

// ---------------------------------------------------------------------------------------------
// Matrix-core variant for 4 query heads per KV head (bf16 or E4M3 caches). The same split-KV
// chunks, exact chunk softmax and partial records as decode_attn_kernel; the dot products run on
// v_mfma_f32_32x32x16_bf16 with the 4 heads padded to the 32 rows of the MFMA (the padding costs
// matrix-core time only, which decode has to spare), so the vector work per cache element drops to
// the E4M3 widening. Each wave takes every fourth block of 32 keys of the chunk.
//  Scores: S[h][key] = sum_d q[h][d] K[key][d]; in K step st, lane half hi covers dims
//  64 hi + 8 st .. + 7, so a lane reads one contiguous half row of its key (B operand) and the
//  heads' q values in the same order (A operand, rows 4..31 zero). Heads land in registers 0..3
//  of lanes 0..31, one key per lane.
//  Output: O[h][d] = sum_key P[h][key] V[key][d]; V rows are staged per wave as bf16 in
//  chunk-swizzled LDS rows and read transposed (ds_read_b64_tr_b16: lane gets keys
//  16 st + {4 hi .. 4 hi + 3, 8 + 4 hi .. 8 + 4 hi + 3} of one dim), and the softmax stores P in
//  that key order, so one 16-byte LDS read per lane gives the A operand.
namespace {
constexpr int kMfRow = 256;                  // LDS bytes per staged bf16 V row
constexpr int kMfTile = 32 * kMfRow;          // one 32-key V block
constexpr int kMfWaveLds = kMfTile;           // one block per wave
__device__ __forceinline__ int mf_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// key of position r (0..15) within a 16-key step of the permuted P order
__device__ __forceinline__ int mf_key(int r) {
  const int hi = r >> 3, j = r & 7;
  return j < 4 ? 4 * hi + j : 8 + 4 * hi + (j - 4);
}
}  // namespace

// At most 256 registers per lane (two workgroups per CU: more loads in flight per CU; the kernel
// fits in ~156 VGPRs, while left unbounded the compiler took 260 and one workgroup per CU).
template <bool FP8>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_mfma_kernel(DecodeParams p) {
  constexpr int G = 4;
  constexpr int kMaxChunk = kDecodeChunkKeys;
  static_assert(kMaxChunk % 32 == 0, "blocks of 32 keys");
  static_assert(G * kMaxChunk >= 4 * G * kHeadDim, "the score rows also hold the final reduction");
  __shared__ float s_s[G * kMaxChunk];
  __shared__ float ml[G][2];
  __shared__ __attribute__((aligned(16))) unsigned char vt[4 * kMfWaveLds];

  // KV heads vary fastest across the grid: the workgroups of one chunk read the same cache rows
  const int kvh = blockIdx.x;
  const int chunk_id = blockIdx.y;
  const int b = blockIdx.z;
  const int pos = p.seqlens[b] - 1;
  if (pos < 0 || (p.window == 0 && pos >= p.rows)) return;
  const int64_t n_valid = min(n_valid_rows(pos, p.window), (int64_t)p.n_chunks * p.chunk);
  const int64_t k0 = (int64_t)chunk_id * p.chunk;
  if (k0 >= n_valid) return;
  const int n = (int)min((int64_t)p.chunk, n_valid - k0);
  const int n_chunks_b = (int)((n_valid + p.chunk - 1) / p.chunk);
  const int n_blk = (n + 31) >> 5;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  constexpr int EB = FP8 ? 1 : 2;                                  // bytes per cache element
  const int64_t row_bytes = (int64_t)p.Hkv * kHeadDim * EB;
  const unsigned char* kc = reinterpret_cast<const unsigned char*>(p.k_cache) +
                            ((int64_t)b * p.rows + k0) * row_bytes + (int64_t)kvh * kHeadDim * EB;
  const unsigned char* vc = reinterpret_cast<const unsigned char*>(p.v_cache) +
                            ((int64_t)b * p.rows + k0) * row_bytes + (int64_t)kvh * kHeadDim * EB;
  const bf16x8 zero8 = bf16x8{};
  unsigned char* wtile = vt + wave * kMfWaveLds;

  // One 32-key block of cache rows: lane pieces of 16 bytes, 16 (bf16) or 8 (E4M3) lanes per row,
  // loaded into registers, then widened and written as bf16 rows of 16 chunks, chunk c at
  // c ^ swz(row). Rows at or past n read as zeros.
  constexpr int NV = FP8 ? 4 : 8;  // 16-byte pieces per lane and block
  // register sets of loaded rows: E4M3 blocks are half the bytes, so a wave keeps its next two
  // in flight; bf16 keeps one (two would cost the occupancy)
  constexpr bool TWO = FP8;
  u32x4 rawA[NV], rawB[NV];
  auto load_rows = [&](u32x4 (&vraw)[NV], const unsigned char* base, int blk) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = 64 * i + lane;
      const int row = FP8 ? (idx >> 3) : (idx >> 4), pc = FP8 ? (idx & 7) : (idx & 15);
      const int key = 32 * blk + row;
      vraw[i] = key < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (int64_t)key * row_bytes) + pc)
                        : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stage_rows = [&](const u32x4 (&vraw)[NV], unsigned char* tile) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = 64 * i + lane;
      if (FP8) {
        const int row = idx >> 3, pc = idx & 7;
        const u32x4 w = vraw[i];
        const u32x4 lo = {e4m3x2_bf16<false>(w[0]), e4m3x2_bf16<true>(w[0]),
                          e4m3x2_bf16<false>(w[1]), e4m3x2_bf16<true>(w[1])};
        const u32x4 up = {e4m3x2_bf16<false>(w[2]), e4m3x2_bf16<true>(w[2]),
                          e4m3x2_bf16<false>(w[3]), e4m3x2_bf16<true>(w[3])};
        *reinterpret_cast<u32x4*>(tile + row * kMfRow + 16 * ((2 * pc) ^ mf_swz(row))) = lo;
        *reinterpret_cast<u32x4*>(tile + row * kMfRow + 16 * ((2 * pc + 1) ^ mf_swz(row))) = up;
      } else {
        const int row = idx >> 4, ch = idx & 15;
        *reinterpret_cast<u32x4*>(tile + row * kMfRow + 16 * (ch ^ mf_swz(row))) = vraw[i];
      }
    }
  };

  // ---- pass A
  {
    bf16x8 qa[8];  // head l32 (< 4), dims 64 hi + 8 st .. + 7
    if (l32 < G) {
      const f32x4* src = reinterpret_cast<const f32x4*>(
          p.qhat + ((int64_t)b * p.Hq + kvh * G + l32) * kHeadDim + 64 * hi);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const f32x4 a = src[2 * st], c = src[2 * st + 1];
        const u32x4 w = {pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(c[0], c[1]),
                         pack_bf16(c[2], c[3])};
        qa[st] = __builtin_bit_cast(bf16x8, w);
      }
    } else {
#pragma unroll
      for (int st = 0; st < 8; ++st) qa[st] = zero8;
    }
    // K rows of this wave's blocks: coalesced row loads (the next block's while the current one
    // is scored), widened to bf16 and staged as swizzled rows; the B operand of K step st is the
    // 16-byte chunk 8 hi + st of row l32
    int kb_off[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) kb_off[st] = l32 * kMfRow + 16 * ((8 * hi + st) ^ mf_swz(l32));
    auto score_block = [&](u32x4 (&vraw)[NV], int blk, int ahead) {
      stage_rows(vraw, wtile);
      if (blk + ahead < n_blk) load_rows(vraw, kc, blk + ahead);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's rows are in LDS
      f32x16 sacc = f32x16{};
#pragma unroll
      for (int st = 0; st < 8; ++st)
        sacc = mfma32(qa[st], *reinterpret_cast<const bf16x8*>(wtile + kb_off[st]), sacc);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the tile is rewritten
      const int key = 32 * blk + l32;
      if (hi == 0 && key < n) {
#pragma unroll
        for (int h = 0; h < G; ++h) s_s[h * kMaxChunk + key] = sacc[h];
      }
    };
    if (wave < n_blk) load_rows(rawA, kc, wave);
    if (TWO) {
      if (wave + 4 < n_blk) load_rows(rawB, kc, wave + 4);
      for (int blk = wave; blk < n_blk; blk += 8) {
        score_block(rawA, blk, 8);
        if (blk + 4 < n_blk) score_block(rawB, blk + 4, 8);
      }
    } else {
      for (int blk = wave; blk < n_blk; blk += 4) score_block(rawA, blk, 4);
    }
  }
  // this wave's first V blocks are loaded while the softmax runs
  if (wave < n_blk) load_rows(rawA, vc, wave);
  if (TWO && wave + 4 < n_blk) load_rows(rawB, vc, wave + 4);
  __syncthreads();

  // ---- exact softmax over the chunk, one wave per head; bf16 P in the permuted key order over
  // the head's score row (dword q = positions 2q, 2q+1 of step q / 8; its keys are >= q, and a
  // later pass of the loop never reads a float an earlier pass wrote)
  const int n_pad = (n + 31) & ~31;
  for (int h = wave; h < G; h += 4) {
    float* sh = s_s + h * kMaxChunk;
    float mx = -INFINITY;
    for (int j = lane; j < n; j += 64) mx = fmaxf(mx, sh[j]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
    const float c = p.scale_log2;
    const float nmc = -mx * c;
    float sum = 0.f;
    for (int q = lane; q < n_pad / 2; q += 64) {
      const int ja = 16 * (q >> 3) + mf_key(2 * (q & 7));
      const int jb = ja + 1;
      const float ea = ja < n ? __builtin_amdgcn_exp2f(__builtin_fmaf(sh[ja], c, nmc)) : 0.f;
      const float eb = jb < n ? __builtin_amdgcn_exp2f(__builtin_fmaf(sh[jb], c, nmc)) : 0.f;
      const uint32_t w = pack_bf16(ea, eb);
      sh[q] = __uint_as_float(w);
      sum += bf16lo(w) + bf16hi(w);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += shfl_xor_f(sum, o);
    if (lane == 0) {
      ml[h][0] = mx * c;
      ml[h][1] = sum;
    }
  }
  __syncthreads();

  // ---- pass B: per 32-key block, stage V as bf16 rows, then two 16-key steps x 4 dim blocks
  int tr_off[2][4];
  {
    const int tr_row = 4 * hi + ((lane & 15) >> 2);
    const int tr_dch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int row = 8 * x + tr_row;
        tr_off[x][db] = row * kMfRow + 16 * ((4 * db + tr_dch) ^ mf_swz(row)) + 8 * (lane & 1);
      }
  }
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  auto pv_block = [&](u32x4 (&vraw)[NV], int blk, int ahead) {
    unsigned char* tile = wtile;
    stage_rows(vraw, tile);
    if (blk + ahead < n_blk) load_rows(vraw, vc, blk + ahead);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's rows are in LDS
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2) {
      const int pstep = 2 * blk + st2;           // 16-key step of the chunk
      bf16x8 pa = zero8;
      if (l32 < G) pa = *reinterpret_cast<const bf16x8*>(s_s + l32 * kMaxChunk + 8 * pstep + 4 * hi);
      const unsigned char* base = tile + st2 * 16 * kMfRow;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const i16x4 a = lds_read_tr(base + tr_off[0][db]);
        const i16x4 c = lds_read_tr(base + tr_off[1][db]);
        const i16x4 both[2] = {a, c};
        o[db] = mfma32(pa, __builtin_bit_cast(bf16x8, both), o[db]);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the tile is rewritten
  };
  if (TWO) {
    for (int blk = wave; blk < n_blk; blk += 8) {
      pv_block(rawA, blk, 8);
      if (blk + 4 < n_blk) pv_block(rawB, blk + 4, 8);
    }
  } else {
    for (int blk = wave; blk < n_blk; blk += 4) pv_block(rawA, blk, 4);
  }
  __syncthreads();  // every wave is done reading P
  float* red = s_s;  // [4 waves][G][128]
  if (hi == 0) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int h = 0; h < G; ++h) red[(wave * G + h) * kHeadDim + 32 * db + l32] = o[db][h];
  }
  __syncthreads();

  const float vs = FP8 ? p.v_scale : 1.0f;
  for (int i = tid; i < G * kHeadDim; i += kDecThreads) {
    const int h = i / kHeadDim;
    const int d = i - h * kHeadDim;
    const float ov = vs * (red[(0 * G + h) * kHeadDim + d] + red[(1 * G + h) * kHeadDim + d] +
                           red[(2 * G + h) * kHeadDim + d] + red[(3 * G + h) * kHeadDim + d]);
    const int head = kvh * G + h;
    if (n_chunks_b == 1) {
      float y = ov / ml[h][1];
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
      rec[4 + d] = ov;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Ring decode in one launch, for 4 query heads per KV head and rings of at most 128 slots (the
// local layers: zh-TW translation page, section 2.3, a fixed 128-token window per sequence). One
// workgroup per (KV head, sequence); wave w owns slots 32 w .. 32 w + 31.
//  1. Every wave issues the loads of its K and V slots at once, beside the new token's rows.
//  2. Wave 0 normalises and rotates the group's 4 q rows, wave 1 the new key row (16 lanes per
//     row, as the prep kernel does); the new k_hat and v go to the cache slot pos % W, and the
//     workgroup keeps the same rows (as the cache holds them) in LDS.
//  3. Scores and output on the matrix cores as in decode_mfma_kernel, the new slot's row taken
//     from LDS instead of the cache (the same workgroup writes that cache row, so reading it back
//     would race); exact softmax over the <= 128 slots, sigmoid gate, bf16 store.
// Results equal the prep + decode_mfma_kernel pair bit for bit (same operand rounding, same
// reduction order).
namespace {
// RMSNorm + RoPE of one 128-dim row held by 16 lanes (lane c: dims 8c .. 8c + 7, w: the norm
// weights of those dims), rotated pairs exchanged through the row's 68-float LDS stage. Result in
// x (fp32).
__device__ __forceinline__ void norm_rope16(float* x, int c, int pos, const float (&w)[8], float eps,
                                            const RopeTable& rt, float* sr) {
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += x[j] * x[j];
  ss = row16_sum(ss);
  const float inv = rsqrtf(ss * (1.0f / kHeadDim) + eps);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] *= inv * w[j];
  const int hr = rt.half;
  if (hr > 0) {
    double rev0 = 0.0, rev1 = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (c == j) {
        rev0 = rt.rev[j];
        rev1 = rt.rev[j + 16];
      }
    }
    const bool rotates = 8 * c < 2 * hr;
    if (rotates) {
      *reinterpret_cast<f32x4*>(sr + 8 * c) = f32x4{x[0], x[1], x[2], x[3]};
      *reinterpret_cast<f32x4*>(sr + 8 * c + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS ops complete in order
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pi = c + 16 * k;
      if (pi < hr) {
        float cs, sn;
        rope_cs(pos, k ? rev1 : rev0, cs, sn);
        const float a = sr[pi];
        const float bb = sr[pi + hr];
        sr[pi] = a * cs - bb * sn;
        sr[pi + hr] = bb * cs + a * sn;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (rotates) {
      const f32x4 lo = *reinterpret_cast<const f32x4*>(sr + 8 * c);
      const f32x4 hi4 = *reinterpret_cast<const f32x4*>(sr + 8 * c + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[j] = lo[j];
        x[4 + j] = hi4[j];
      }
    }
  }
}
}  // namespace

template <bool FP8>
__global__ __launch_bounds__(kDecThreads) void decode_ring_kernel(DecodeParams p) {
  constexpr int G = 4;
  constexpr int kSlots = 128;
  __shared__ float s_s[G * kSlots];
  __shared__ float ml[G][2];
  __shared__ __attribute__((aligned(16))) unsigned char vt[4 * kMfWaveLds];
  __shared__ __attribute__((aligned(16))) uint32_t qhs[G][64];   // bf16 q_hat rows
  __shared__ __attribute__((aligned(16))) uint32_t newk[64];     // new slot's K row (bf16)
  __shared__ __attribute__((aligned(16))) uint32_t newv[64];     // new slot's V row (bf16)
  __shared__ __attribute__((aligned(16))) float stage[G + 1][kDpStage];

  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const int W = p.window;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  constexpr int EB = FP8 ? 1 : 2;
  const int64_t row_bytes = (int64_t)p.Hkv * kHeadDim * EB;
  const unsigned char* kc = reinterpret_cast<const unsigned char*>(p.k_cache) +
                            (int64_t)b * W * row_bytes + (int64_t)kvh * kHeadDim * EB;
  const unsigned char* vc = reinterpret_cast<const unsigned char*>(p.v_cache) +
                            (int64_t)b * W * row_bytes + (int64_t)kvh * kHeadDim * EB;
  const bf16x8 zero8 = bf16x8{};
  unsigned char* wtile = vt + wave * kMfWaveLds;

  constexpr int NV = FP8 ? 4 : 8;
  // every slot below W is read (the ring holds W rows whatever the position), so the loads need
  // not wait for the sequence length; rows at or past the valid count are zeroed once it is known
  // The ring holds W rows whatever the position, so the loads need not wait for the sequence
  // length: a buffer resource spanning slots 0 .. W-1 of this (sequence, KV head) returns zeros
  // for slots at or past W without a per-lane branch; rows at or past the valid count are zeroed
  // once the length is known.
  auto load_rows = [&](u32x4 (&vraw)[NV], const unsigned char* base, int blk) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)base, 0, (int)((int64_t)(W - 1) * row_bytes + kHeadDim * EB), 0x00020000);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = 64 * i + lane;
      const int row = FP8 ? (idx >> 3) : (idx >> 4), pc = FP8 ? (idx & 7) : (idx & 15);
      const int key = 32 * blk + row;
      vraw[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, key * (int)row_bytes + 16 * pc, 0, 2));
    }
  };
  auto zero_past = [&](u32x4 (&vraw)[NV], int blk, int n_valid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = 64 * i + lane;
      const int row = FP8 ? (idx >> 3) : (idx >> 4);
      if (32 * blk + row >= n_valid) vraw[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto stage_rows = [&](const u32x4 (&vraw)[NV], unsigned char* tile) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = 64 * i + lane;
      if (FP8) {
        const int row = idx >> 3, pc = idx & 7;
        const u32x4 w = vraw[i];
        const u32x4 lo = {e4m3x2_bf16<false>(w[0]), e4m3x2_bf16<true>(w[0]),
                          e4m3x2_bf16<false>(w[1]), e4m3x2_bf16<true>(w[1])};
        const u32x4 up = {e4m3x2_bf16<false>(w[2]), e4m3x2_bf16<true>(w[2]),
                          e4m3x2_bf16<false>(w[3]), e4m3x2_bf16<true>(w[3])};
        *reinterpret_cast<u32x4*>(tile + row * kMfRow + 16 * ((2 * pc) ^ mf_swz(row))) = lo;
        *reinterpret_cast<u32x4*>(tile + row * kMfRow + 16 * ((2 * pc + 1) ^ mf_swz(row))) = up;
      } else {
        const int row = idx >> 4, ch = idx & 15;
        *reinterpret_cast<u32x4*>(tile + row * kMfRow + 16 * (ch ^ mf_swz(row))) = vraw[i];
      }
    }
  };
  // the new slot's row (bf16 words in LDS) over its row of this wave's tile, if the slot is here
  auto put_new_row = [&](const uint32_t* src, unsigned char* tile, int new_slot) {
    const int r = new_slot - 32 * wave;
    if (r >= 0 && r < 32 && lane < 16) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(src + 4 * lane);
      *reinterpret_cast<u32x4*>(tile + r * kMfRow + 16 * (lane ^ mf_swz(r))) = w;
    }
  };

  // ---- 1. every load the workgroup needs goes out first, none waiting on another: the new
  // token's rows (q: wave 0, k: wave 1 lanes 0..15, v: wave 1 lanes 16..31) and the gate logits of
  // the output elements this thread writes, then this wave's cache slots (the new slot's stale row
  // is replaced below), then the sequence length. Loads complete in issue order, so the new rows,
  // issued first, are normalised while the cache rows are still in flight.
  const int grp = lane >> 4, c = lane & 15;
  const bool is_q = wave == 0;
  u32x4 xnew = u32x4{0u, 0u, 0u, 0u};
  if (wave == 0 || (wave == 1 && grp < 2)) {
    const uint16_t* src = is_q ? p.q_new + ((int64_t)b * p.Hq + kvh * G + grp) * kHeadDim
                        : grp == 0 ? p.k_new + ((int64_t)b * p.Hkv + kvh) * kHeadDim
                                   : p.v_new + ((int64_t)b * p.Hkv + kvh) * kHeadDim;
    xnew = *reinterpret_cast<const u32x4*>(src + 8 * c);
  }
  float wv[8];  // norm weights of this lane's 8 dims of the new q or k row
  {
    const float* w = is_q ? p.q_norm_w : p.k_norm_w;
    if (w) {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + 8 * c);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + 8 * c + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wv[j] = w0[j];
        wv[4 + j] = w1[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = 1.0f;
    }
  }
  // this thread writes output elements 2 tid and 2 tid + 1 of the group's 4 x 128; their gate
  // logits come as one word (read from the q rows, of the same shape, when ungated, and unused)
  static_assert(G * kHeadDim == 2 * kDecThreads, "two output elements per thread");
  const int64_t out_base = ((int64_t)b * p.Hq + kvh * G) * kHeadDim + 2 * tid;
  const uint32_t graw = *reinterpret_cast<const uint32_t*>((p.gated ? p.gate : p.q_new) + out_base);
  u32x4 kraw[NV], vraw[NV];  // waves past the ring's W slots read zeros
  load_rows(kraw, kc, wave);
  load_rows(vraw, vc, wave);
  // A length below 1 is a caller error: the workgroup then computes on position 0 and writes
  // nothing (no early exit, which would let the compiler sink the loads above behind this read).
  const int pos_raw = p.seqlens[b] - 1;
  const bool valid = pos_raw >= 0;
  const int pos = valid ? pos_raw : 0;
  const int n = min(pos + 1, W);   // valid slots 0 .. n-1 (positions max(0, pos-W+1) .. pos)
  const int slot = pos % W;        // the new token's slot
  const int n_blk = (n + 31) >> 5;

  // ---- 2. the new token: q rows (wave 0), k row (wave 1, lanes 0..15), v row (wave 1, 16..31)
  {
    if (wave == 0 || (wave == 1 && grp == 0)) {
      float x[8];
      unpack8(xnew, x);
      norm_rope16(x, c, pos, wv, p.eps, p.rope, &stage[is_q ? grp : G][0]);
      if (is_q) {
        *reinterpret_cast<u32x4*>(&qhs[grp][4 * c]) = pack8(x);
      } else {
        const int64_t off = ((int64_t)b * W + slot) * p.Hkv * kHeadDim + (int64_t)kvh * kHeadDim + 8 * c;
        if (!FP8) {
          const u32x4 w = pack8(x);
          if (valid) *reinterpret_cast<u32x4*>(p.k_cache + off) = w;
          *reinterpret_cast<u32x4*>(&newk[4 * c]) = w;
        } else {
          const float ki = p.k_inv;
          const u32x2 w = {pack4_e4m3(x[0] * ki, x[1] * ki, x[2] * ki, x[3] * ki),
                           pack4_e4m3(x[4] * ki, x[5] * ki, x[6] * ki, x[7] * ki)};
          if (valid) *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(p.k_cache) + off) = w;
          *reinterpret_cast<u32x4*>(&newk[4 * c]) =
              u32x4{e4m3x2_bf16<false>(w[0]), e4m3x2_bf16<true>(w[0]), e4m3x2_bf16<false>(w[1]),
                    e4m3x2_bf16<true>(w[1])};
        }
      }
    } else if (wave == 1 && grp == 1) {
      const u32x4 vw = xnew;
      const int64_t off = ((int64_t)b * W + slot) * p.Hkv * kHeadDim + (int64_t)kvh * kHeadDim + 8 * c;
      if (!FP8) {
        if (valid) *reinterpret_cast<u32x4*>(p.v_cache + off) = vw;
        *reinterpret_cast<u32x4*>(&newv[4 * c]) = vw;
      } else {
        float vf[8];
        unpack8(vw, vf);
        const float vi = p.v_inv;
        const u32x2 w = {pack4_e4m3(vf[0] * vi, vf[1] * vi, vf[2] * vi, vf[3] * vi),
                         pack4_e4m3(vf[4] * vi, vf[5] * vi, vf[6] * vi, vf[7] * vi)};
        if (valid) *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(p.v_cache) + off) = w;
        *reinterpret_cast<u32x4*>(&newv[4 * c]) =
            u32x4{e4m3x2_bf16<false>(w[0]), e4m3x2_bf16<true>(w[0]), e4m3x2_bf16<false>(w[1]),
                  e4m3x2_bf16<true>(w[1])};
      }
    }
  }
  __syncthreads();

  // ---- 3a. scores of this wave's 32 slots
  if (wave < n_blk) {
    bf16x8 qa[8];
#pragma unroll
    for (int st = 0; st < 8; ++st)
      qa[st] = l32 < G ? *reinterpret_cast<const bf16x8*>(&qhs[l32][32 * hi + 4 * st]) : zero8;
    zero_past(kraw, wave, n);
    stage_rows(kraw, wtile);
    put_new_row(newk, wtile, slot);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's rows are in LDS
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int st = 0; st < 8; ++st)
      sacc = mfma32(qa[st], *reinterpret_cast<const bf16x8*>(wtile + l32 * kMfRow + 16 * ((8 * hi + st) ^ mf_swz(l32))), sacc);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the tile is rewritten
    const int key = 32 * wave + l32;
    if (hi == 0 && key < n) {
#pragma unroll
      for (int h = 0; h < G; ++h) s_s[h * kSlots + key] = sacc[h];
    }
  }
  __syncthreads();

  // ---- 3b. exact softmax over the slots, one wave per head; bf16 P in the permuted key order
  // over the head's score row (a single pass: n / 2 <= 64 words)
  {
    const int h = wave;
    float* sh = s_s + h * kSlots;
    float mx = -INFINITY;
    for (int j = lane; j < n; j += 64) mx = fmaxf(mx, sh[j]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
    const float c = p.scale_log2;
    const float nmc = -mx * c;
    const int n_pad = (n + 31) & ~31;
    float sum = 0.f;
    const int q = lane;
    uint32_t w = 0;
    if (q < n_pad / 2) {
      const int ja = 16 * (q >> 3) + mf_key(2 * (q & 7));
      const int jb = ja + 1;
      const float ea = ja < n ? __builtin_amdgcn_exp2f(__builtin_fmaf(sh[ja], c, nmc)) : 0.f;
      const float eb = jb < n ? __builtin_amdgcn_exp2f(__builtin_fmaf(sh[jb], c, nmc)) : 0.f;
      w = pack_bf16(ea, eb);
      sum = bf16lo(w) + bf16hi(w);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // every lane's reads precede the writes
    if (q < n_pad / 2) sh[q] = __uint_as_float(w);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += shfl_xor_f(sum, o);
    if (lane == 0) {
      ml[h][0] = mx * c;
      ml[h][1] = sum;
    }
  }
  __syncthreads();

  // ---- 3c. output of this wave's 32 slots: two 16-key steps x 4 dim blocks
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  if (wave < n_blk) {
    int tr_off[2][4];
    const int tr_row = 4 * hi + ((lane & 15) >> 2);
    const int tr_dch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int row = 8 * x + tr_row;
        tr_off[x][db] = row * kMfRow + 16 * ((4 * db + tr_dch) ^ mf_swz(row)) + 8 * (lane & 1);
      }
    zero_past(vraw, wave, n);
    stage_rows(vraw, wtile);
    put_new_row(newv, wtile, slot);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int st2 = 0; st2 < 2; ++st2) {
      const int pstep = 2 * wave + st2;
      bf16x8 pa = zero8;
      if (l32 < G) pa = *reinterpret_cast<const bf16x8*>(s_s + l32 * kSlots + 8 * pstep + 4 * hi);
      const unsigned char* base = wtile + st2 * 16 * kMfRow;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const i16x4 a = lds_read_tr(base + tr_off[0][db]);
        const i16x4 cc = lds_read_tr(base + tr_off[1][db]);
        const i16x4 both[2] = {a, cc};
        o[db] = mfma32(pa, __builtin_bit_cast(bf16x8, both), o[db]);
      }
    }
  }
  __syncthreads();  // every wave is done with its tile and with P
  float* red = reinterpret_cast<float*>(vt);  // [4 waves][G][128]
  if (hi == 0) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int h = 0; h < G; ++h) red[(wave * G + h) * kHeadDim + 32 * db + l32] = o[db][h];
  }
  __syncthreads();

  const float vs = FP8 ? p.v_scale : 1.0f;
  {
    const int h = (2 * tid) / kHeadDim;
    const int d = 2 * tid - h * kHeadDim;
    float y[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float ov = vs * (red[(0 * G + h) * kHeadDim + d + e] + red[(1 * G + h) * kHeadDim + d + e] +
                             red[(2 * G + h) * kHeadDim + d + e] + red[(3 * G + h) * kHeadDim + d + e]);
      y[e] = ov / ml[h][1];
      if (p.gated) {
        const float g = e ? bf16hi(graw) : bf16lo(graw);
        y[e] *= __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
      }
    }
    if (valid) *reinterpret_cast<uint32_t*>(p.out + out_base) = pack_bf16(y[0], y[1]);
  }
}

// bf16 -> E4M3 of value * inv_scale, 16 elements per lane.
__global__ __launch_bounds__(256) void to_fp8_kernel(ToFp8Params p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i * 16 >= p.n) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(p.src + 16 * i);
  float x[16];
  unpack8(s[0], x);
  unpack8(s[1], x + 8);
  *reinterpret_cast<u32x4*>(p.dst + 16 * i) = pack16_e4m3(x, p.inv_scale);
}

hipError_t launch_to_fp8(const ToFp8Params& p, hipStream_t s) {
  const int64_t lanes = p.n / 16;
  if (lanes == 0) return hipSuccess;
  hipLaunchKernelGGL(to_fp8_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

// One workgroup per (head, sequence), one thread per output dim. The chunk weights exp2(m_c - M)
// are formed once (chunks spread over the threads) and shared through LDS; the per-dim sums then
// issue their loads independently of each other.
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeParams p) {
  __shared__ float w_s[kDecodeMaxChunks];
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
  // even chunks sum into o0, odd ones into o1, in chunk order; sixteen chunks' loads are issued
  // together so the loop waits on memory once per sixteen chunks rather than once per two
  float o0 = 0.f, o1 = 0.f;
  int c = 0;
  for (; c + 15 < nc; c += 16) {
    float r[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = rec[(int64_t)(c + i) * kPartStride + 4 + d];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      o0 += r[i] * w_s[c + i];
      o1 += r[i + 1] * w_s[c + i + 1];
    }
  }
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

// ---------------------------------------------------------------------------------------------
// Device-resident scratch for callers that cannot allocate (zg_attn_decode_noalloc): the decode
// workspace (fp32 q_hat and the split-KV partials) lives in this array, one copy per GPU, for the
// life of the process. Host code never passes the array's name to a kernel: on the host it is a
// stand-in symbol, not a device address. The device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept per device.
static __device__ __attribute__((aligned(256))) unsigned char decode_scratch[kDecodeScratchBytes];

hipError_t decode_scratch_ptr(void** out) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void* ptr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev]() {
    void* a = nullptr;
    err[dev] = hipGetSymbolAddress(&a, HIP_SYMBOL(decode_scratch));
    ptr[dev] = a;
  });
  if (err[dev] != hipSuccess) return err[dev];
  *out = ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  if (p.window > 0 && p.window <= 128 && p.Hq == 4 * p.Hkv) {
    if (p.fp8) hipLaunchKernelGGL(decode_ring_kernel<true>, dim3(p.Hkv, p.B), dim3(kDecThreads), 0, s, p);
    else hipLaunchKernelGGL(decode_ring_kernel<false>, dim3(p.Hkv, p.B), dim3(kDecThreads), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(decode_prep_kernel, dim3((unsigned)(((int64_t)p.B * (p.Hq + p.Hkv) + 15) / 16)),
                     dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = p.Hq / p.Hkv;
  const dim3 grid(p.n_chunks, p.Hkv, p.B);
  const dim3 grid_h(p.Hkv, p.n_chunks, p.B);
  switch (G * 2 + (p.fp8 ? 1 : 0)) {
    case 2: hipLaunchKernelGGL(decode_attn_kernel<1>, grid, dim3(kDecThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL(decode_attn_kernel<2>, grid, dim3(kDecThreads), 0, s, p); break;
    case 8: hipLaunchKernelGGL(decode_mfma_kernel<false>, grid_h, dim3(kDecThreads), 0, s, p); break;
    case 16: hipLaunchKernelGGL(decode_attn_kernel<8>, grid, dim3(kDecThreads), 0, s, p); break;
    case 3: hipLaunchKernelGGL(decode_attn_fp8_kernel<1>, grid, dim3(kDecThreads), 0, s, p); break;
    case 5: hipLaunchKernelGGL(decode_attn_fp8_kernel<2>, grid, dim3(kDecThreads), 0, s, p); break;
    case 9: hipLaunchKernelGGL(decode_mfma_kernel<true>, grid_h, dim3(kDecThreads), 0, s, p); break;
    case 17: hipLaunchKernelGGL(decode_attn_fp8_kernel<8>, grid, dim3(kDecThreads), 0, s, p); break;
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
