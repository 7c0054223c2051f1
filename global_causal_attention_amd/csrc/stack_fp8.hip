// E4M3 projections of one Pre-LN attention layer. The pages run the model's matrix
// multiplications in FP8 with the E4M3 format on the forward pass (ZGCM-1 zh-TW translation page,
// section 3.1, pre-training setup); here that format carries the q/k/v/gate and output
// projections: the normalised hidden state and the attention output become E4M3 rows with one
// fp32 scale per row, the weights E4M3 rows (one scale per output channel), and the GEMM
// Y = diag(sx) (Xq Wq^T) diag(sw) runs on the gfx950 FP8 matrix cores with fp32 accumulation.
//
// Quantization of a row h: scale = amax / 448 and codes = E4M3(h * (448 / amax)), each factor
// rounded to fp32 once, the codes rounded to nearest-even and saturated at +-448; a row of zeros
// gets scale 1 and zero codes.
#include "zg_common.hpp"

namespace zg {

namespace {
constexpr int kQThreads = 256;   // one workgroup of 4 waves per row
constexpr int kQMaxPer = 4;      // 8-element groups per thread: dim <= 8 * 256 * 4 = 8192

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, shfl_xor_f(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += shfl_xor_f(v, o);
  return v;
}

// The row's codes and scale from the thread's groups h[i] (group g = tid + 256 i, valid for
// g < n_grp); `red` is 4 floats of LDS. Every thread of the workgroup calls it.
__device__ __forceinline__ void quant_row_store(float (&h)[kQMaxPer][8], int n_grp, uint8_t* y,
                                                float* y_scale, float* red) {
  const int tid = threadIdx.x;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kQMaxPer; ++i)
    if (tid + kQThreads * i < n_grp)
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(h[i][j]));
  amax = wave_max(amax);
  __syncthreads();  // `red` may still hold an earlier reduction
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.f ? 448.0f / amax : 0.f;
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < kQMaxPer; ++i) {
    const int g = tid + kQThreads * i;
    if (g < n_grp) {
      const u32x2 w = {pack4_e4m3(h[i][0] * inv, h[i][1] * inv, h[i][2] * inv, h[i][3] * inv),
                       pack4_e4m3(h[i][4] * inv, h[i][5] * inv, h[i][6] * inv, h[i][7] * inv)};
      *reinterpret_cast<u32x2*>(y + 8 * g) = w;
    }
  }
  if (tid == 0) *y_scale = scale;
}
}  // namespace

// ---------------------------------------------------------------------------------------------
// E4M3 rows of RMSNorm(x) * w: h = (x / sqrt(mean(x^2) + eps)) * w in fp32, then quantized.
__global__ __launch_bounds__(kQThreads) void rmsnorm_fp8_kernel(RmsNormFp8Params p) {
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const float* x = p.x + r * p.dim;
  const int tid = threadIdx.x;
  const int n_grp = p.dim / 8;
  float h[kQMaxPer][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kQMaxPer; ++i) {
    const int g = tid + kQThreads * i;
    if (g < n_grp) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(x + 8 * g);
      const f32x4 b = *reinterpret_cast<const f32x4*>(x + 8 * g + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[i][j] = a[j];
        h[i][4 + j] = b[j];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) ss += h[i][j] * h[i][j];
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float inv = rsqrtf(tot / (float)p.dim + p.eps);
#pragma unroll
  for (int i = 0; i < kQMaxPer; ++i) {
    const int g = tid + kQThreads * i;
    if (g < n_grp) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h[i][j] *= inv;
        if (p.w) h[i][j] *= p.w[8 * g + j];
      }
    }
  }
  quant_row_store(h, n_grp, p.y + r * p.dim, p.y_scale + r, red);
}

// E4M3 rows of bf16 rows (row stride ldx elements).
__global__ __launch_bounds__(kQThreads) void quant_rows_kernel(QuantRowsParams p) {
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const uint16_t* x = p.x + r * p.ldx;
  const int tid = threadIdx.x;
  const int n_grp = p.dim / 8;
  float h[kQMaxPer][8];
#pragma unroll
  for (int i = 0; i < kQMaxPer; ++i) {
    const int g = tid + kQThreads * i;
    if (g < n_grp) unpack8(*reinterpret_cast<const u32x4*>(x + 8 * g), h[i]);
  }
  quant_row_store(h, n_grp, p.y + r * p.dim, p.y_scale + r, red);
}

hipError_t launch_rmsnorm_fp8(const RmsNormFp8Params& p, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_fp8_kernel, dim3((unsigned)p.rows), dim3(kQThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const QuantRowsParams& p, hipStream_t s) {
  hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)p.rows), dim3(kQThreads), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// E4M3 GEMM: Y[m, n] = sx[m] sw[n] sum_k X[m, k] W[n, k], both operands K-contiguous bytes. The
// tile scheme of the bf16 GEMM, one byte per element: one workgroup of 8 waves (two per SIMD)
// computes a 256 x 256 tile, each wave a 128 x 64 block of 4 x 2 blocks of
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, unit block scales), so an X operand read from
// LDS feeds two MFMAs and a W operand four, and one wave's stage loads and barrier waits overlap
// the other's MFMAs. K advances 128 per stage: 256 rows of 128 bytes of
// X and of W stream into LDS by buffer_load ... lds, double-buffered, one barrier per stage; a
// stage is two 64-deep MFMA steps. A lane's 32 operand bytes of a step are two 16-byte chunks of
// its row, the same k positions for both operands (the MFMA sums over whatever k each element
// pair stands for, so only the pairing has to agree). Chunks are XOR-swizzled by (row / 2 mod 8)
// as in the bf16 GEMM, and the tiles are ordered per XCD in groups of 8 m-tiles.
namespace {
constexpr int kFBM = 256;                    // tile M
constexpr int kFBN = 256;                    // tile N
constexpr int kFBK = 128;                    // K per stage = bytes per staged row
constexpr int kFNBuf = 2;                    // stages resident in LDS
constexpr int kFThreads = 512;               // 8 waves
constexpr int kFRowsPerDma = 1024 / kFBK;    // rows filled by one DMA instruction (1 KB)
constexpr int kFDmaPerSlab = kFBM / kFRowsPerDma / 8;  // DMA instructions per wave per slab
constexpr int kFTileA = kFBM * kFBK;
constexpr int kFStage = kFTileA + kFBN * kFBK;
constexpr int kFLds = kFNBuf * kFStage;
constexpr int kFGroupM = 8;
constexpr int kFSub = kFBK / 64;             // MFMA steps per stage
static_assert(kFLds <= 160 * 1024, "LDS budget");

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int fswz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8 a, const i32x8 b, const f32x16 c) {
  // cbsz = blgp = 0: both operands E4M3; block scales 127 (E8M0 for 1.0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
}  // namespace

__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_fp8_kernel(GemmFp8Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- tile of this workgroup (XCD-contiguous ranges, groups of 8 m-tiles per n-tile column)
  const int n_tn = (p.N + kFBN - 1) / kFBN;
  const int64_t n_tm = (p.M + kFBM - 1) / kFBM;
  const int64_t n_tiles = n_tm * n_tn;
  int64_t t = blockIdx.x;
  if (n_tiles % 8 == 0) t = (t % 8) * (n_tiles / 8) + t / 8;
  const int64_t per_group = (int64_t)kFGroupM * n_tn;
  const int64_t grp = t / per_group;
  const int64_t first_m = grp * kFGroupM;
  const int gm = (int)min((int64_t)kFGroupM, n_tm - first_m);
  const int64_t rr = t - grp * per_group;
  // tile indices made visibly wave-uniform (the DMA takes its buffer resource in SGPRs)
  const int64_t m0 = (int64_t)__builtin_amdgcn_readfirstlane((int)(first_m + rr % gm)) * kFBM;
  const int n0 = __builtin_amdgcn_readfirstlane((int)(rr / gm)) * kFBN;

  // ---- stage DMA: wave w fills DMA groups [w, w + 1) * kFDmaPerSlab of each slab
  const uint32_t rowb = (uint32_t)p.K;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.x + m0 * p.K), 0, (int)(min(p.M - m0, (int64_t)kFBM) * rowb), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.w + (int64_t)n0 * p.K), 0, (int)(min(p.N - n0, kFBN) * rowb), 0x00020000);
  // lane -> row lane / 8 of the DMA group, physical chunk lane % 8
  const int dr = lane >> 3;
  const int dp = lane & 7;
  const uint32_t voff0 = dr * rowb + 16 * (dp ^ fswz(dr));
  const uint32_t voff1 = dr * rowb + 16 * (dp ^ fswz(dr + kFRowsPerDma));
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  auto dma_stage = [&](int buf, int k0) {
    const uint32_t base = lds0 + buf * kFStage + wave * kFDmaPerSlab * 1024;
    const uint32_t s0 = wave * kFDmaPerSlab * kFRowsPerDma * rowb + k0;
#pragma unroll
    for (int i = 0; i < kFDmaPerSlab; ++i) {
      const uint32_t soff = s0 + i * kFRowsPerDma * rowb;
      const uint32_t voff = (i & 1) ? voff1 : voff0;
      lds_dma16(base + i * 1024, voff, ra, soff);
      lds_dma16(base + kFTileA + i * 1024, voff, rb, soff);
    }
  };

  // ---- operand reads: row (block + 32 i + l32), logical chunks 4 ks + 2 hi and 4 ks + 2 hi + 1
  const int wm = (wave >> 2) * 128;
  const int wn = (wave & 3) * 64;
  int a_off[kFSub][2], b_off[kFSub][2];
#pragma unroll
  for (int ks = 0; ks < kFSub; ++ks)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int c = 16 * ((4 * ks + 2 * hi + h2) ^ fswz(l32));
      a_off[ks][h2] = (wm + l32) * kFBK + c;
      b_off[ks][h2] = kFTileA + (wn + l32) * kFBK + c;
    }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int n_k = p.K / kFBK;
  dma_stage(0, 0);
  for (int it = 0; it < n_k; ++it) {
    // this stage's DMA has landed; the barrier publishes every wave's and guarantees that all
    // reads of the buffer refilled next (stage it - 1) are done
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (it + 1 < n_k) dma_stage((it + 1) % kFNBuf, (it + 1) * kFBK);
    const unsigned char* st = smem + (it % kFNBuf) * kFStage;
    i32x8 a[2][4], b[2][2];
    auto rd = [&](const int (&off)[kFSub][2], int ks, int i) -> i32x8 {
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(st + off[ks][0] + 32 * kFBK * i);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(st + off[ks][1] + 32 * kFBK * i);
      return i32x8{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                   (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
    };
    // The first MFMAs need only the step's four B operands and one A operand; every further A
    // operand (and the next step's operands) is read while the MFMAs of the row block before it
    // run, so little of the stage's read volume stands in front of idle matrix cores.
#pragma unroll
    for (int j = 0; j < 2; ++j) b[0][j] = rd(b_off, 0, j);
    a[0][0] = rd(a_off, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kFSub; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i + 1 < 4) {
          a[ks][i + 1] = rd(a_off, ks, i + 1);
        } else if (ks + 1 < kFSub) {
#pragma unroll
          for (int j = 0; j < 2; ++j) b[ks + 1][j] = rd(b_off, ks + 1, j);
          a[ks + 1][0] = rd(a_off, ks + 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma_fp8(a[ks][i], b[ks][j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // ---- epilogue: lane holds column n = l32 of each 32x32 block, rows 8*(r/4) + 4*hi + r%4.
  // Row block by row block: the block's accumulators take their rows' and columns' scales (no
  // branches, so the loops unroll and the accumulators stay in registers), then the store as in the
  // bf16 GEMM; one block's row scales at a time keeps the epilogue within 256 registers.
  float ws[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn + 32 * j + l32;
    ws[j] = p.w_scale[min(n, p.N - 1)];
  }
  const bool full = m0 + kFBM <= p.M && n0 + kFBN <= p.N;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t mb = m0 + wm + 32 * i + 4 * hi;
    float xs[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) xs[r] = p.x_scale[min(mb + 8 * (r >> 2) + (r & 3), p.M - 1)];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] *= xs[r] * ws[j];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + l32;
      if (full) {
        if (p.residual) {
          float* rp = p.residual + mb * p.N + n;
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = rp[(int64_t)(8 * (r >> 2) + (r & 3)) * p.N];
#pragma unroll
          for (int r = 0; r < 16; ++r) rp[(int64_t)(8 * (r >> 2) + (r & 3)) * p.N] = v[r] + acc[i][j][r];
        }
        if (p.y) {
          uint16_t* yp = p.y + mb * p.ldy + n;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            yp[(int64_t)(8 * (r >> 2) + (r & 3)) * p.ldy] = (uint16_t)(pack_bf16(acc[i][j][r], 0.f) & 0xffffu);
        }
        continue;
      }
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = mb + 8 * (r >> 2) + (r & 3);
        if (m >= p.M) continue;
        const float v = acc[i][j][r];
        if (p.residual) p.residual[m * p.N + n] += v;
        if (p.y) p.y[m * p.ldy + n] = (uint16_t)(pack_bf16(v, 0.f) & 0xffffu);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

hipError_t launch_gemm_fp8(const GemmFp8Params& p, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_fp8_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kFLds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((p.M + kFBM - 1) / kFBM) * ((p.N + kFBN - 1) / kFBN);
  hipLaunchKernelGGL(gemm_fp8_kernel, dim3((unsigned)tiles), dim3(kFThreads), kFLds, s, p);
  return hipGetLastError();
}

}  // namespace zg
