// Building blocks of one Pre-LN attention layer with projections (ZGCM-1 zh-TW translation page,
// section 2.1 and Figure 3: a normalised hidden state feeds parallel q/k/v/gate projections, o_proj
// follows; section 3.1 names Pre-LN): a row RMSNorm (fp32 residual in, bf16 out) and a bf16 MFMA
// GEMM Y = X W^T with an optional fp32 residual-accumulate epilogue.
#include "zg_common.hpp"

namespace zg {

// ---------------------------------------------------------------------------------------------
// RMSNorm over rows of an fp32 matrix; one 256-thread block per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(RmsNormParams p) {
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const float* x = p.x + r * p.dim;
  uint16_t* y = p.y + r * p.dim;
  const int tid = threadIdx.x;
  float ss = 0.f;
  for (int i = 8 * tid; i < p.dim; i += 8 * 256) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(x + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(x + i + 4);
    ss += a[0] * a[0] + a[1] * a[1] + a[2] * a[2] + a[3] * a[3];
    ss += b[0] * b[0] + b[1] * b[1] + b[2] * b[2] + b[3] * b[3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += shfl_xor_f(ss, o);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = rsqrtf(tot / (float)p.dim + p.eps);
  for (int i = 8 * tid; i < p.dim; i += 8 * 256) {
    float v[8];
    const f32x4 a = *reinterpret_cast<const f32x4*>(x + i);
    const f32x4 b = *reinterpret_cast<const f32x4*>(x + i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j] * inv;
      v[4 + j] = b[j] * inv;
    }
    if (p.w) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] *= p.w[i + j];
    }
    *reinterpret_cast<u32x4*>(y + i) = pack8(v);
  }
}

hipError_t launch_rmsnorm(const RmsNormParams& p, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)p.rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// GEMM: Y[m, n] = sum_k X[m, k] W[n, k]. Both operands are K-contiguous, so each MFMA operand lane
// reads 16 contiguous bytes of a row from LDS. 128 x 128 tile per 256-thread workgroup, each wave a
// 64 x 64 quadrant of 2 x 2 v_mfma_f32_32x32x16_bf16 blocks; K advances 64 per stage with register
// prefetch and two LDS buffers.
namespace {
constexpr int kGT = 128;          // tile M and N
constexpr int kGK = 64;           // K per stage
constexpr int kGRow = 144;        // LDS bytes per 64-element row (+16 pad, conflict-free)
constexpr int kGTile = kGT * kGRow;
constexpr int kGBuf = 2 * kGTile;

__device__ __forceinline__ f32x16 mfma32g(const bf16x8 a, const bf16x8 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
}  // namespace

__global__ __launch_bounds__(256) void gemm_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int n_tiles_n = (p.N + kGT - 1) / kGT;
  const int64_t tm = blockIdx.x / n_tiles_n;
  const int tn = blockIdx.x - (int)(tm * n_tiles_n);
  const int64_t m0 = tm * kGT;
  const int n0 = tn * kGT;
  const int wm = (wave >> 1) * 64;
  const int wn = (wave & 1) * 64;

  // loader: each thread moves 4 x 16 B of X and of W per stage: row = tid / 2, 64-byte half.
  const int lrow = tid >> 1;
  const int lhalf = tid & 1;
  const bool xrow_ok = m0 + lrow < p.M;
  const bool wrow_ok = n0 + lrow < p.N;
  const uint16_t* xsrc = p.x + (xrow_ok ? (m0 + lrow) : 0) * (int64_t)p.K + 32 * lhalf;
  const uint16_t* wsrc = p.w + (int64_t)(wrow_ok ? (n0 + lrow) : 0) * p.K + 32 * lhalf;
  u32x4 px[4], pw[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      px[j] = xrow_ok ? *reinterpret_cast<const u32x4*>(xsrc + k0 + 8 * j) : u32x4{0u, 0u, 0u, 0u};
      pw[j] = wrow_ok ? *reinterpret_cast<const u32x4*>(wsrc + k0 + 8 * j) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int buf) {
    unsigned char* xs = smem + buf * kGBuf;
    unsigned char* ws = xs + kGTile;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<u32x4*>(xs + lrow * kGRow + 64 * lhalf + 16 * j) = px[j];
      *reinterpret_cast<u32x4*>(ws + lrow * kGRow + 64 * lhalf + 16 * j) = pw[j];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int n_k = p.K / kGK;
  load(0);
  store(0);
  __syncthreads();
  for (int it = 0; it < n_k; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_k) load((it + 1) * kGK);
    const unsigned char* xs = smem + buf * kGBuf;
    const unsigned char* ws = xs + kGTile;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8*>(xs + (wm + 32 * i + l32) * kGRow + 32 * ks + 16 * hi);
        bb[i] = *reinterpret_cast<const bf16x8*>(ws + (wn + 32 * i + l32) * kGRow + 32 * ks + 16 * hi);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32g(a[i], bb[j], acc[i][j]);
    }
    if (it + 1 < n_k) store(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column n = l32 of each 32x32 block, rows 8*(r/4) + 4*hi + r%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + l32;
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (m >= p.M) continue;
        const float v = acc[i][j][r];
        if (p.residual) p.residual[m * p.N + n] += v;
        if (p.y) p.y[m * p.ldy + n] = (uint16_t)(pack_bf16(v, 0.f) & 0xffffu);
      }
    }
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  constexpr int lds = 2 * kGBuf;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((p.M + kGT - 1) / kGT) * ((p.N + kGT - 1) / kGT);
  hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)tiles), dim3(256), lds, s, p);
  return hipGetLastError();
}

}  // namespace zg
