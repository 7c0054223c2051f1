// Prefill attention for gfx950: banded (sliding-window) or full causal GQA attention with a fused
// QK-RMSNorm + partial-RoPE prologue on q, bf16 MFMA for QK^T and PV, online softmax in fp32 and the
// sigmoid gate fused into the epilogue.
//
// Method: ZGCM-1 zh-TW translation page, section 2.1 "Model overview" and Figure 3 (GQA 32/8 heads of
// dim 128, 128-token window on local layers, full causal attention on global layers, QK-RMSNorm,
// partial RoPE, GatedSWA(h) = o_proj(A_SWA(q,k,v) * sigmoid(g_proj(h)))).
//
// Work decomposition. One workgroup = 8 waves = one (sequence b, KV head) and a tile of queries for
// all G query heads that share that KV head, so every K/V tile staged in LDS serves G heads. Wave w
// owns query head (w % G) and 32 consecutive queries (block w / G): Mq = 256 / G queries per tile.
// Keys stream in tiles of 64; each tile is loaded into registers one iteration ahead and written to
// one of two LDS buffers, so one barrier per tile suffices.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16). Scores are computed transposed, S^T = K Q^T
// (A = 32 keys x 16 dims from LDS, B = Q^T from registers), so each lane owns one query and 16 of the
// 32 keys of a block; row max/sum need one lane-pair exchange. O^T = V^T P^T reuses the score
// registers directly as the B operand: within each 16-key step the lane's keys are {0-3, 8-11} or
// {4-7, 12-15}, so V is stored transposed in LDS with bits 2 and 3 of the key index swapped, which
// makes each lane's 8 A-operand values one contiguous 16-byte LDS read. O^T keeps one query per lane,
// so the online-softmax rescale is a per-lane scalar.
#include "zg_common.hpp"

namespace zg {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kNk = 64;                     // keys per tile
constexpr int kRow = 256;                   // LDS bytes per K or V row (unpadded, chunk-swizzled)
constexpr int kTileBytes = kNk * kRow;      // 16384
constexpr int kQWaveBytes = 32 * kRow;      // per-wave q staging: 32 chunk-swizzled rows
// LDS: two K buffers, then two V buffers. q staging aliases them before the first tile.
constexpr int kLdsK0 = 0;
constexpr int kLdsV0 = 2 * kTileBytes;
constexpr int kLdsBytes = 4 * kTileBytes;
static_assert(kWaves * kQWaveBytes <= kLdsBytes, "q staging aliases the K/V buffers");

// 16-byte chunk c of tile row r is stored at chunk c ^ swz(r). Sixteen consecutive rows read at one
// logical chunk (the QK^T operand) and four aligned rows read at four adjacent chunks (the transposed
// V operand) both land on distinct banks.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

__device__ __forceinline__ f32x16 mfma32(const bf16x8 a, const bf16x8 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element (i % 4) of the 8-byte
// rows addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12.
__device__ __forceinline__ i16x4 lds_read_tr(const unsigned char* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// K prologue: khat[b,t,h,:] = bf16(RoPE(RMSNorm(k[b,t,h,:]))), packed [B, T, Hkv, 128].
// Two lanes per row; 128 rows per 256-thread block.
__global__ __launch_bounds__(256) void kprep_kernel(KPrepParams p) {
  __shared__ float stage[128 * 64];
  const int lane_pair = threadIdx.x >> 1;
  const int half = threadIdx.x & 1;
  const int64_t row = (int64_t)blockIdx.x * 128 + lane_pair;
  const int64_t n_rows = (int64_t)p.B * p.T * p.Hkv;
  if (row >= n_rows) return;  // rows come in lane pairs, so both lanes of a pair exit together
  const int64_t bt = row / p.Hkv;
  const int h = (int)(row - bt * p.Hkv);
  const int t = (int)(bt % p.T);
  const uint16_t* src = p.k + bt * p.sk + (int64_t)h * kHeadDim + 64 * half;
  float x[64];
  const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int i = 0; i < 8; ++i) unpack8(s4[i], x + 8 * i);
  norm_rope_row(x, half, p.k_norm_w, p.eps, p.pos0 + t, p.rope, stage, lane_pair, 128);
  u32x4* d4 = reinterpret_cast<u32x4*>(p.khat + row * kHeadDim + 64 * half);
#pragma unroll
  for (int i = 0; i < 8; ++i) d4[i] = pack8(x + 8 * i);
}

// ---------------------------------------------------------------------------------------------
template <int G, bool GATED>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  constexpr int QB = kWaves / G;   // 32-query blocks per head
  constexpr int MQ = 32 * QB;      // queries per tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- work item: heavy query tiles first for full causal attention
  const int per_tile = p.B * p.Hkv;
  const int t_idx = blockIdx.x / per_tile;
  const int bh = blockIdx.x - t_idx * per_tile;
  const int qtile = (p.window == 0) ? (p.n_qtiles - 1 - t_idx) : t_idx;
  const int b = bh / p.Hkv;
  const int kvh = bh - b * p.Hkv;
  const int r0 = qtile * MQ;
  const int T = p.T;
  const int W = p.window;

  const int hg = wave % G;
  const int qb = wave / G;
  const int head = kvh * G + hg;
  const int qbase = r0 + 32 * qb;

  // ---- q prologue: wave-private staging (32 chunk-swizzled rows of 256 B, aliasing K/V buffers)
  bf16x8 qf[8];
  {
    unsigned char* qs = smem + wave * 32 * kRow;
    const int r = lane >> 1;
    const int half = lane & 1;
    const int t = qbase + r;
    float x[64];
    if (t < T) {
      const u32x4* s4 = reinterpret_cast<const u32x4*>(
          p.q + ((int64_t)b * T + t) * p.sq + (int64_t)head * kHeadDim + 64 * half);
#pragma unroll
      for (int i = 0; i < 8; ++i) unpack8(s4[i], x + 8 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] = 0.f;
    }
    // the [dim][row] RoPE scratch (32 rows x 64 floats) overlays this wave's staging rows; every
    // access to it precedes the bf16 row writes below in this wave's program order
    norm_rope_row(x, half, p.q_norm_w, p.eps, p.pos0 + t, p.rope, reinterpret_cast<float*>(qs), r,
                  32);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(qs + r * kRow + 16 * ((8 * half + i) ^ swz(r))) = pack8(x + 8 * i);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(qs + l32 * kRow + 16 * ((2 * s + hi) ^ swz(l32)));
    __syncthreads();
  }

  // ---- key tile range of the workgroup
  const int q_last = min(r0 + MQ, T) - 1;
  int k_begin = 0;
  if (W > 0) k_begin = max(0, r0 - W + 1) & ~(kNk - 1);
  const int n_tiles = (q_last + 1 - k_begin + kNk - 1) / kNk;

  // ---- ping-pong schedule. Waves 0-3 (group A) and 4-7 (group B) each hold one wave per SIMD
  // and run one phase apart, so in every phase between two barriers one wave of each SIMD issues
  // MFMAs (QK^T of tile j and PV of tile j-1) while the other runs the softmax of its tile on the
  // vector ALUs. During its softmax phase a group streams the next tile it owns straight from
  // memory into LDS (group A: K tiles, group B: V tiles):
  //   phase 2j   : A MFMA(j)                  B softmax(j-1), loads V_j     (read from 2j+2)
  //   phase 2j+1 : A softmax(j), loads K_{j+1} (read from 2j+2)   B MFMA(j)
  // Two K and two V buffers; a buffer is refilled only after its last reader's phase ended.
  const bool grp_b = wave >= 4;
  const int wg = wave & 3;
  const int dma_row = 16 * wg + (lane >> 4);       // + 4 i, i = 0..3
  const int dma_pch = lane & 15;                   // physical chunk this lane fills
  const uint16_t* g_src = grp_b ? p.v + (int64_t)b * T * p.sv + (int64_t)kvh * kHeadDim
                                : p.khat + ((int64_t)b * T * p.Hkv + kvh) * kHeadDim;
  const int64_t g_rstride = grp_b ? p.sv : (int64_t)p.Hkv * kHeadDim;
  const int buf0 = grp_b ? kLdsV0 : kLdsK0;

  auto dma_tile = [&](int t) {  // rows past the end are clamped to row T-1 (in bounds)
    const int kt = k_begin + t * kNk;
    unsigned char* dst = smem + buf0 + (t & 1) * kTileBytes + 16 * wg * kRow;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = dma_row + 4 * i;
      const int key = min(kt + row, T - 1);
      const uint16_t* src = g_src + (int64_t)key * g_rstride + 8 * (dma_pch ^ swz(row));
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(dst + 4 * i * kRow),
                                       16, 0, 0);
    }
  };
  // V rows past the end must read as zero (their weights are zero, and 0 * Inf would be NaN)
  auto zero_tail = [&](int t) {
    const int kt = k_begin + t * kNk;
    if (grp_b && kt + kNk > T) {
      __builtin_amdgcn_s_waitcnt(0);
      unsigned char* dst = smem + buf0 + (t & 1) * kTileBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = dma_row + 4 * i;
        if (kt + row >= T)
          *reinterpret_cast<u32x4*>(dst + row * kRow + 16 * dma_pch) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // ---- running softmax state: one query per lane; lanes l and l^32 share the query. The maximum
  // is only raised when a tile exceeds it by more than 2^8 in exp2 units (lazy rescale), so
  // unnormalised weights stay <= 256.
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = -1e30f;
  float l_run = 0.f;
  const float c = p.scale_log2;
  const int my_q = qbase + l32;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  f32x16 s[2];
  uint32_t pk[2][8];

  // A operands of one MFMA phase, in issue order: 16 QK^T operands (K rows, st-major, both key
  // blocks) then 16 PV operands (V^T via two transposing reads each, st-major, four dim blocks).
  const int tr_row = 4 * hi + ((lane & 15) >> 2);          // + 16 st + 8 x
  const int tr_dch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // + 4 db: logical 16-B chunk
  const int tr_sub = 8 * (lane & 1);
  auto operand = [&](int j, int i) -> bf16x8 {
    if (i < 16) {
      const int st = i >> 1, kb = i & 1;
      const int row = 32 * kb + l32;
      return *reinterpret_cast<const bf16x8*>(smem + kLdsK0 + (j & 1) * kTileBytes + row * kRow +
                                              16 * ((2 * st + hi) ^ swz(row)));
    }
    const int st = (i - 16) >> 2, db = (i - 16) & 3;
    const unsigned char* vb = smem + kLdsV0 + ((j - 1) & 1) * kTileBytes;
    const int r_a = 16 * st + tr_row;
    const int r_b = r_a + 8;
    const int ch = 4 * db + tr_dch;
    const i16x4 a = lds_read_tr(vb + r_a * kRow + 16 * (ch ^ swz(r_a)) + tr_sub);
    const i16x4 bb = lds_read_tr(vb + r_b * kRow + 16 * (ch ^ swz(r_b)) + tr_sub);
    const i16x4 both[2] = {a, bb};
    return __builtin_bit_cast(bf16x8, both);
  };
  auto qk_only = [&](int j) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int st = i >> 1, kb = i & 1;
      s[kb] = mfma32(operand(j, i), qf[st], s[kb]);
    }
  };
  auto mfma_phase = [&](int j) {  // j >= 1: S = K_j Q^T, then O^T += V_{j-1}^T P^T
    constexpr int kAhead = 8;
    bf16x8 ring[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) ring[i] = operand(j, i);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const bf16x8 a = ring[i % kAhead];
      if (i < 16) {
        const int st = i >> 1, kb = i & 1;
        s[kb] = mfma32(a, qf[st], s[kb]);
      } else {
        const int st = (i - 16) >> 2, db = (i - 16) & 3;
        const int kb = st >> 1, h8 = (st & 1) * 4;
        u32x4 bw = {pk[kb][h8], pk[kb][h8 + 1], pk[kb][h8 + 2], pk[kb][h8 + 3]};
        o[db] = mfma32(a, __builtin_bit_cast(bf16x8, bw), o[db]);
      }
      if (i + kAhead < 32) ring[i % kAhead] = operand(j, i + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto final_pv = [&](int j) {  // O^T += V_j^T P^T
#pragma unroll
    for (int i = 16; i < 32; ++i) {
      const int st = (i - 16) >> 2, db = (i - 16) & 3;
      const int kb = st >> 1, h8 = (st & 1) * 4;
      u32x4 bw = {pk[kb][h8], pk[kb][h8 + 1], pk[kb][h8 + 2], pk[kb][h8 + 3]};
      o[db] = mfma32(operand(j + 1, i), __builtin_bit_cast(bf16x8, bw), o[db]);
    }
  };
  auto softmax_phase = [&](int j) {  // S -> P (bf16, packed), running max / sum
    const int kt = k_begin + j * kNk;
    const bool need_mask = (kt + kNk - 1 > qbase) || ((W > 0) && (kt < qbase + 31 - W + 1));
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = (key <= my_q) && (W == 0 || key > my_q - W);
          s[kb][r] = ok ? s[kb][r] : -INFINITY;
        }
    }
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    {  // partner lane l ^ 32 holds the other keys of the same query (VALU lane swap, no LDS)
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(mx, __uint_as_float(hi ? sw[0] : sw[1]));
    }
    if (__builtin_amdgcn_ballot_w64((mx - m_run) * c > 8.0f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
    }
    const float mc = m_run * c;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c, -mc));
        pk[kb][r >> 1] = pack_bf16(p0, p1);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[kb][r >> 1]), ones, rs,
                                             false);
      }
    l_run += rs;
  };

  // ---- preamble: A streams K_0, B streams V_0
  dma_tile(0);
  zero_tail(0);
  __syncthreads();
  if (grp_b) __syncthreads();  // B starts one phase behind
  for (int j = 0; j < n_tiles; ++j) {
    if (j == 0) qk_only(0);
    else mfma_phase(j);
    __syncthreads();
    softmax_phase(j);
    if (j + 1 < n_tiles) {
      dma_tile(j + 1);
      zero_tail(j + 1);
    }
    __syncthreads();
  }
  final_pv(n_tiles - 1);
  if (!grp_b) __syncthreads();  // matches B's extra barrier

  // ---- epilogue: normalise, gate, round, store (one query per lane, 4 dims per store)
  if (my_q < T) {
    const float l_tot = l_run + shfl_xor_f(l_run, 32);
    const float inv = 1.0f / l_tot;
    const int64_t tok = (int64_t)b * T + my_q;
    uint16_t* dst = p.out + tok * p.so + (int64_t)head * kHeadDim;
    const uint16_t* gsrc = GATED ? p.gate + tok * p.sg + (int64_t)head * kHeadDim : nullptr;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * db + 8 * rq + 4 * hi;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = o[db][4 * rq + j] * inv;
        if (GATED) {
          const u32x2 g = *reinterpret_cast<const u32x2*>(gsrc + d0);
          const float gv[4] = {bf16lo(g[0]), bf16hi(g[0]), bf16lo(g[1]), bf16hi(g[1])};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            y[j] *= __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv[j] * 1.4426950408889634f));
        }
        u32x2 w = {pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
        *reinterpret_cast<u32x2*>(dst + d0) = w;
      }
  }
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_kprep(const KPrepParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.T * p.Hkv;
  const int64_t blocks = (rows + 127) / 128;
  hipLaunchKernelGGL(kprep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int G, bool GATED>
static hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s) {
  constexpr int lds = kLdsBytes;
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = prefill_kernel<G, GATED>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int64_t grid = (int64_t)p.n_qtiles * p.B * p.Hkv;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, int group, bool gated, hipStream_t s) {
  switch (group * 2 + (gated ? 1 : 0)) {
    case 2: return launch_prefill_t<1, false>(p, s);
    case 3: return launch_prefill_t<1, true>(p, s);
    case 4: return launch_prefill_t<2, false>(p, s);
    case 5: return launch_prefill_t<2, true>(p, s);
    case 8: return launch_prefill_t<4, false>(p, s);
    case 9: return launch_prefill_t<4, true>(p, s);
    case 16: return launch_prefill_t<8, false>(p, s);
    case 17: return launch_prefill_t<8, true>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace zg
