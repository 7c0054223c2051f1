// Device helpers shared by the gfx950 kernels: bf16 packing, vector types, wave shuffles, and the
// fused QK-RMSNorm + partial-RoPE row prologue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zg_kernels.hpp"

namespace zg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kMaxRotHalf = 32;  // rot_dim <= 64

// Rotary frequencies in revolutions per position (theta_i / (2 pi), fp64, computed on the host).
typedef RopeTableH RopeTable;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to nearest-even bf16 and pack (lo in bits 0..15): v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ void unpack8(const u32x4 w, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16lo(w[i]);
    x[2 * i + 1] = bf16hi(w[i]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float* x) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
  return w;
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Value of lane ^ 1 (DPP quad permutation [1, 0, 3, 2]; VALU only).
__device__ __forceinline__ float dpp_swap_pair(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF,
                                                             0xF, false));
}

// One LDS-direct load (buffer_load_dwordx4 ... lds): lane l's 16 bytes at buffer offset
// voff + soff go to LDS byte address lds + 16 l, so one instruction fills 1 KB of consecutive LDS.
// Issued in inline asm so that the compiler's wait tracking does not make later LDS reads wait
// for it (callers wait with explicit vmcnt counts). m0, which carries the LDS address, is saved
// and restored inside the statement, and one wait state separates its write from the load.
__device__ __forceinline__ void lds_dma16(uint32_t lds, uint32_t voff, __amdgpu_buffer_rsrc_t rsrc,
                                          uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

// cos/sin of 2*pi*(pos * rev). The product is reduced modulo one revolution in fp64, so the angle
// keeps full precision at positions up to 2^18 and beyond; v_sin_f32 / v_cos_f32 take their input
// in revolutions (max abs error ~1.2e-7 on [-0.5, 0.5]).
__device__ __forceinline__ void rope_cs(int64_t pos, double rev, float& c, float& s) {
  double r = (double)pos * rev;
  r = r - __builtin_rint(r);
  const float a = (float)r;
  s = __builtin_amdgcn_sinf(a);
  c = __builtin_amdgcn_cosf(a);
}

// Fused QK-RMSNorm + partial RoPE of one 128-wide head row, split over two adjacent lanes:
// lane parity `half` holds dims [64*half, 64*half + 64) in x[0..63] (fp32, already loaded).
// RMSNorm: x * w / sqrt(mean(x^2) + eps) over all 128 dims (partner lane = lane ^ 1).
// RoPE: pairs (i, i + rot/2), i < rot/2 <= 32, all inside half 0, rotated by pos * theta_i.
// `stage` is LDS scratch laid out [dim][row] with `stride` rows (this lane pair is `row`), so lanes
// of consecutive rows hit consecutive banks; only half 0 touches it.
__device__ __forceinline__ void norm_rope_row(float* x, int half, const float* __restrict__ w,
                                              float eps, int64_t pos, const RopeTable& rt,
                                              float* stage, int row, int stride) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) ss += x[i] * x[i];
  ss += shfl_xor_f(ss, 1);
  const float inv = rsqrtf(ss * (1.0f / kHeadDim) + eps);
  if (w) {
    const f32x4* w4 = reinterpret_cast<const f32x4*>(w + 64 * half);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      f32x4 ww = w4[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * i + j] *= inv * ww[j];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] *= inv;
  }
  const int h = rt.half;
  if (half == 0 && h > 0) {
    float* st = stage + row;
#pragma unroll
    for (int i = 0; i < 64; ++i)
      if (i < 2 * h) st[i * stride] = x[i];
#pragma unroll
    for (int i = 0; i < kMaxRotHalf; ++i) {
      if (i < h) {
        float c, s;
        rope_cs(pos, rt.rev[i], c, s);
        const float a = st[i * stride];
        const float b = st[(i + h) * stride];
        st[i * stride] = a * c - b * s;
        st[(i + h) * stride] = b * c + a * s;
      }
    }
#pragma unroll
    for (int i = 0; i < 64; ++i)
      if (i < 2 * h) x[i] = st[i * stride];
  }
}

// Variant of norm_rope_row for kernels that keep loads in flight across the prologue: the weights
// are read through scalar loads of both halves (the lane picks its half), so the prologue issues no
// vector-memory instruction that would wait behind those loads. `scale` multiplies the result.
typedef __attribute__((address_space(4))) const float* const_f32_ptr;
__device__ __forceinline__ void norm_rope_row_scalar_w(float* x, int half, const_f32_ptr w,
                                                       float eps, float scale, int64_t pos,
                                                       const RopeTable& rt, float* stage, int row,
                                                       int stride) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) ss += x[i] * x[i];
  ss += shfl_xor_f(ss, 1);
  const float inv = rsqrtf(ss * (1.0f / kHeadDim) + eps) * scale;
  if (w) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      float wl = w[i], wh = w[64 + i];
      asm("" : "+s"(wl), "+s"(wh));  // keep both as scalar loads; the lane selects its half
      x[i] *= inv * (half ? wh : wl);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) x[i] *= inv;
  }
  const int h = rt.half;
  if (half == 0 && h > 0) {
    float* st = stage + row;
#pragma unroll
    for (int i = 0; i < 64; ++i)
      if (i < 2 * h) st[i * stride] = x[i];
#pragma unroll
    for (int i = 0; i < kMaxRotHalf; ++i) {
      if (i < h) {
        float c, s;
        rope_cs(pos, rt.rev[i], c, s);
        const float a = st[i * stride];
        const float b = st[(i + h) * stride];
        st[i * stride] = a * c - b * s;
        st[(i + h) * stride] = b * c + a * s;
      }
    }
#pragma unroll
    for (int i = 0; i < 64; ++i)
      if (i < 2 * h) x[i] = st[i * stride];
  }
}

// E4M3 (OCP 8-bit float: 4 exponent bits, bias 7, 3 mantissa bits, largest finite 448): four
// floats rounded to nearest-even E4M3 codes, saturated to +-448 first (the conversion itself turns
// values beyond the range into NaN), packed in element order.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  const uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, -448.f, 448.f),
                                                     __builtin_amdgcn_fmed3f(b, -448.f, 448.f), 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, -448.f, 448.f),
                                         __builtin_amdgcn_fmed3f(d, -448.f, 448.f), w, true);
}

}  // namespace zg
