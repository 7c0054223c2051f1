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
constexpr int kKRow = 272;                  // LDS bytes per K row (256 + 16 pad: conflict-free)
constexpr int kVtRow = 144;                 // LDS bytes per V^T row (128 + 16 pad)
constexpr int kKBytes = kNk * kKRow;        // 17408
constexpr int kVtBytes = kHeadDim * kVtRow; // 18432
constexpr int kBufBytes = kKBytes + kVtBytes;
constexpr int kQRow = 272;
constexpr int kQWaveBytes = 32 * kQRow;     // per-wave q staging (8704)
static_assert(kWaves * kQWaveBytes <= 2 * kBufBytes, "q staging aliases the K/V buffers");

__device__ __forceinline__ f32x16 mfma32(const bf16x8 a, const bf16x8 b, const f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Swap bits 2 and 3 of a key index inside its 16-key group (an involution).
__device__ __forceinline__ int vt_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
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
  norm_rope_row(x, half, p.k_norm_w, p.eps, p.pos0 + t, p.rope, stage + 64 * lane_pair);
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

  // ---- q prologue: wave-private staging rows (aliasing the K/V buffers)
  bf16x8 qf[8];
  {
    unsigned char* qs = smem + wave * kQWaveBytes;
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
    norm_rope_row(x, half, p.q_norm_w, p.eps, p.pos0 + t, p.rope,
                  reinterpret_cast<float*>(qs + r * kQRow));
    u32x4* d4 = reinterpret_cast<u32x4*>(qs + r * kQRow + 128 * half);
#pragma unroll
    for (int i = 0; i < 8; ++i) d4[i] = pack8(x + 8 * i);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(qs + l32 * kQRow + 32 * s + 16 * hi);
    __syncthreads();
  }

  // ---- key tile range of the workgroup
  const int q_last = min(r0 + MQ, T) - 1;
  int k_begin = 0;
  if (W > 0) k_begin = max(0, r0 - W + 1) & ~(kNk - 1);
  const int k_end = q_last + 1;  // exclusive
  const int n_tiles = (k_end - k_begin + kNk - 1) / kNk;

  // ---- loader mapping: threads 0..255 stage V^T (4 keys x 8 dims), 256..511 stage K (1 row x 64 B)
  const bool v_loader = tid < 256;
  const int lt = tid & 255;
  const int v_kq = lt & 15;          // key quad
  const int v_dc = lt >> 4;          // dim chunk of 8
  const int k_row = lt >> 2;         // 0..63
  const int k_ch = lt & 3;           // 64-byte chunk
  u32x4 pre[4];

  auto load_tile = [&](int kt) {
    if (v_loader) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = kt + 4 * v_kq + j;
        if (key < T) {
          pre[j] = *reinterpret_cast<const u32x4*>(
              p.v + ((int64_t)b * T + key) * p.sv + (int64_t)kvh * kHeadDim + 8 * v_dc);
        } else {
          pre[j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    } else {
      const int key = kt + k_row;
      if (key < T) {
        const u32x4* src = reinterpret_cast<const u32x4*>(
            p.khat + (((int64_t)b * T + key) * p.Hkv + kvh) * kHeadDim + 32 * k_ch);
#pragma unroll
        for (int j = 0; j < 4; ++j) pre[j] = src[j];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) pre[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* base = smem + buf * kBufBytes;
    if (v_loader) {
      unsigned char* vt = base + kKBytes;
      const int pq = (v_kq & ~3) | ((v_kq & 1) << 1) | ((v_kq >> 1) & 1);  // vt_pos(4*kq)/4
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x2 w;
        w[0] = __builtin_amdgcn_perm(pre[1][wi], pre[0][wi], sel);
        w[1] = __builtin_amdgcn_perm(pre[3][wi], pre[2][wi], sel);
        *reinterpret_cast<u32x2*>(vt + (8 * v_dc + e) * kVtRow + pq * 8) = w;
      }
    } else {
      u32x4* dst = reinterpret_cast<u32x4*>(base + k_row * kKRow + 64 * k_ch);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = pre[j];
    }
  };

  // ---- running softmax state (one query per lane; lanes l and l^32 share the query)
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m_run = -1e30f;
  float l_run = 0.f;
  const float c = p.scale_log2;
  const int my_q = qbase + l32;

  if (n_tiles > 0) {
    load_tile(k_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int kt = k_begin + it * kNk;
    const int buf = it & 1;
    if (it + 1 < n_tiles) load_tile(kt + kNk);

    // wave-level relevance of this tile
    const bool after_all = kt > qbase + 31;
    const bool before_all = (W > 0) && (kt + kNk - 1 < qbase - W + 1);
    if (!after_all && !before_all) {
      const unsigned char* kl = smem + buf * kBufBytes;
      const unsigned char* vt = kl + kKBytes;
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(kl + (32 * kb + l32) * kKRow + 32 * st + 16 * hi);
          s[kb] = mfma32(a, qf[st], s[kb]);
        }
      }
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
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      const float mc = m_new * c;
      float rs = 0.f;
      uint32_t pk[2][8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c, -mc));
          rs += p0 + p1;
          pk[kb][r >> 1] = pack_bf16(p0, p1);
        }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= alpha;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kb = st >> 1;
        const int h8 = (st & 1) * 4;
        u32x4 bw = {pk[kb][h8], pk[kb][h8 + 1], pk[kb][h8 + 2], pk[kb][h8 + 3]};
        const bf16x8 bop = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(vt + (32 * db + l32) * kVtRow + 32 * st + 16 * hi);
          o[db] = mfma32(a, bop, o[db]);
        }
      }
    }
    if (it + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

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
  constexpr int lds = 2 * kBufBytes;
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
