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
// reads 16 contiguous bytes of a staged row. One workgroup of 8 waves (two per SIMD) computes a
// 256 x 256 tile; each wave owns a 128 x 64 block of 4 x 2 v_mfma_f32_32x32x16_bf16 blocks, so an X
// operand read from LDS feeds two MFMAs and a W operand four. Two waves per SIMD let one wave's
// stage loads and barrier waits overlap the other's MFMAs (with one wave per SIMD and 128 x 128
// blocks the operand reads halve but the matrix cores idle whenever that wave waits: ~10% slower). K advances 64 per stage: the stage's 256-row X and
// W slabs (128 bytes per row) stream into LDS by buffer_load ... lds, double-buffered, one barrier
// per stage; within a stage the operands of the next 16-deep step are read while the 16 MFMAs of
// the current one run. A staged row keeps its eight 16-byte chunks XOR-swizzled by (row / 2 mod 8): two
// 128-byte rows share one 256-byte bank window, so the 16 rows of one read pass then cover all 64
// banks exactly once; the DMA realises the swizzle by permuting the global addresses of the lanes
// (the LDS side of one DMA instruction is 1 KB of consecutive bytes = 8 whole rows). Rows past M or N read as zeros through the buffer range check.
// Tiles are ordered for L2 reuse: workgroup i runs on XCD i mod 8, so each XCD is given a
// contiguous range of tiles, walked in groups of 8 m-tiles sharing one n-tile column at a time.
namespace {
constexpr int kGBM = 256;                   // tile M
constexpr int kGBN = 256;                   // tile N
constexpr int kGBK = 64;                    // K per stage (32 or 64)
constexpr int kGNBuf = 2;                   // stages resident in LDS
constexpr int kGThreads = 512;              // 8 waves
constexpr int kGRowB = 2 * kGBK;            // bytes per staged row
constexpr int kGChunks = kGRowB / 16;       // 16-byte chunks per staged row
constexpr int kGRowsPerDma = 1024 / kGRowB; // rows filled by one DMA instruction (1 KB)
constexpr int kGDmaPerSlab = kGBM / kGRowsPerDma / 8;  // DMA instructions per wave per slab
constexpr int kGTileA = kGBM * kGRowB;
constexpr int kGStage = kGTileA + kGBN * kGRowB;
constexpr int kGLds = kGNBuf * kGStage;
constexpr int kGGroupM = 8;
static_assert(kGBK == 32 || kGBK == 64, "stage depth");
static_assert(kGLds <= 160 * 1024, "LDS budget");

// Physical chunk of logical chunk c in staged row r: the rows sharing one 256-byte bank window
// differ in (r mod (256 / row bytes)), the XOR term enumerates the rest of a 16-row read pass.
__device__ __forceinline__ int gswz(int r) {
  return kGBK == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

__device__ __forceinline__ f32x16 mfma32g(const bf16x8 a, const bf16x8 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
}  // namespace

__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- tile of this workgroup
  const int n_tn = (p.N + kGBN - 1) / kGBN;
  const int64_t n_tm = (p.M + kGBM - 1) / kGBM;
  const int64_t n_tiles = n_tm * n_tn;
  int64_t t = blockIdx.x;
  if (n_tiles % 8 == 0) t = (t % 8) * (n_tiles / 8) + t / 8;
  const int64_t per_group = (int64_t)kGGroupM * n_tn;
  const int64_t grp = t / per_group;
  const int64_t first_m = grp * kGGroupM;
  const int gm = (int)min((int64_t)kGGroupM, n_tm - first_m);
  const int64_t rr = t - grp * per_group;
  const int64_t m0 = (first_m + rr % gm) * kGBM;
  const int n0 = (int)(rr / gm) * kGBN;

  // ---- stage DMA: wave w fills DMA groups [w, w + 1) * kGDmaPerSlab of each slab
  const uint32_t rowb = (uint32_t)p.K * 2;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.x + m0 * p.K), 0, (int)(min(p.M - m0, (int64_t)kGBM) * rowb), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.w + (int64_t)n0 * p.K), 0, (int)(min(p.N - n0, kGBN) * rowb), 0x00020000);
  // lane -> row lane / kGChunks of the DMA group, physical chunk lane % kGChunks; the logical
  // chunk depends on the group's parity only through gswz (64-deep stages, odd groups)
  const int dr = lane / kGChunks;
  const int dp = lane % kGChunks;
  const uint32_t voff0 = dr * rowb + 16 * (dp ^ gswz(dr));
  const uint32_t voff1 = dr * rowb + 16 * (dp ^ gswz(dr + kGRowsPerDma));
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  auto dma_stage = [&](int buf, int k0) {
    const uint32_t base = lds0 + buf * kGStage + wave * kGDmaPerSlab * 1024;
    const uint32_t s0 = wave * kGDmaPerSlab * kGRowsPerDma * rowb + 2 * k0;
#pragma unroll
    for (int i = 0; i < kGDmaPerSlab; ++i) {
      const uint32_t soff = s0 + i * kGRowsPerDma * rowb;
      const uint32_t voff = (i & 1) ? voff1 : voff0;
      lds_dma16(base + i * 1024, voff, ra, soff);
      lds_dma16(base + kGTileA + i * 1024, voff, rb, soff);
    }
  };

  // ---- operand reads: row (quadrant + 32 i + l32), logical chunk 2 ks + hi
  const int wm = (wave >> 2) * 128;
  const int wn = (wave & 3) * 64;
  constexpr int kSub = kGBK / 16;
  int a_off[kSub], b_off[kSub];
#pragma unroll
  for (int ks = 0; ks < kSub; ++ks) {
    const int c = 16 * ((2 * ks + hi) ^ gswz(l32));
    a_off[ks] = (wm + l32) * kGRowB + c;
    b_off[ks] = kGTileA + (wn + l32) * kGRowB + c;
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int n_k = p.K / kGBK;
  for (int s = 0; s < kGNBuf - 1 && s < n_k; ++s) dma_stage(s, s * kGBK);
  for (int it = 0; it < n_k; ++it) {
    // this wave's DMA of stage it has landed (later stages may still be in flight); the barrier
    // publishes every wave's and guarantees that all reads of the buffer refilled next (stage
    // it - 1) are done
    const int ahead = min(kGNBuf - 2, n_k - 1 - it);  // stages issued after stage it
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | ((4 * kGDmaPerSlab) & 15) | (((4 * kGDmaPerSlab) >> 4) << 14));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * kGDmaPerSlab) & 15) | (((2 * kGDmaPerSlab) >> 4) << 14));
    else __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (it + kGNBuf - 1 < n_k) dma_stage((it + kGNBuf - 1) % kGNBuf, (it + kGNBuf - 1) * kGBK);
    const unsigned char* st = smem + (it % kGNBuf) * kGStage;
    // operands of step ks + 1 are read while the 16 MFMAs of step ks run
    bf16x8 a[2][4], b[2][2];
    auto read_ops = [&](int ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[ks & 1][i] = *reinterpret_cast<const bf16x8*>(st + a_off[ks] + 32 * kGRowB * i);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[ks & 1][j] = *reinterpret_cast<const bf16x8*>(st + b_off[ks] + 32 * kGRowB * j);
    };
    read_ops(0);
#pragma unroll
    for (int ks = 0; ks < kSub; ++ks) {
      if (ks + 1 < kSub) read_ops(ks + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32g(a[ks & 1][i], b[ks & 1][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue: lane holds column n = l32 of each 32x32 block, rows 8*(r/4) + 4*hi + r%4.
  // Full tiles issue a block's 16 residual loads before any add or store.
  const bool full = m0 + kGBM <= p.M && n0 + kGBN <= p.N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + l32;
      const int64_t mb = m0 + wm + 32 * i + 4 * hi;
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
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kGLds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((p.M + kGBM - 1) / kGBM) * ((p.N + kGBN - 1) / kGBN);
  hipLaunchKernelGGL(gemm_kernel, dim3((unsigned)tiles), dim3(kGThreads), kGLds, s, p);
  return hipGetLastError();
}

}  // namespace zg
